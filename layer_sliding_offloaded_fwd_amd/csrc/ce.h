// Chunked LM-head cross-entropy launcher.
#pragma once
#include "common.h"

namespace slide {

int ce_check(const slide_ce_cfg* c, int N);
size_t ce_workspace_bytes(const slide_ce_cfg& c, int N);
int ce_n_chunks(const slide_ce_cfg& c);
int ce_stats(const slide_ce_cfg& c, const void* h, const void* w, const int32_t* tgt, int N,
             int ci, void* ws, hipStream_t st);
int ce_loss(const slide_ce_cfg& c, const int32_t* tgt, int N, float* loss, void* ws,
            hipStream_t st);
int ce_grad(const slide_ce_cfg& c, const void* h, const void* w, const int32_t* tgt, int N,
            int ci, bool with_dh, void* dw, void* ws, hipStream_t st);
int ce_dh(const slide_ce_cfg& c, int N, void* dh, void* ws, hipStream_t st);
int ce_run(const slide_ce_cfg& c, const void* h, const void* w, const int32_t* tgt, int N,
           float* loss, void* dh, void* dw, void* ws, hipStream_t st);

}  // namespace slide
