// Greedy next-token choice for the generation loop: the argmax of each row of
// the head's logits ("Full Forward Pass", How it works: a generation loop
// feeds the chosen token back; the greedy choice is the most likely token),
// either over full fp32 logits rows or over the (value, column) partials the
// head product leaves when it reduces its tiles itself (EpiArgmax).
// Ties go to the lowest index; NaN logits are never chosen over a number.
#include "kernels.h"

namespace gpt2 {

constexpr int kArgmaxThreads = 256;

GPT2_DEV bool argmax_better(float v, int i, float w, int j) { return w > v || (w == v && j < i); }

// The workgroup's best (value, column) over its threads' candidates, then the
// token written for sequence b: the row's next id and column `step` of out.
GPT2_DEV void argmax_finish(float best, int bi, int V, int b, int32_t* __restrict__ next_ids,
                            int32_t* __restrict__ out, int out_stride, int step) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float bits = __int_as_float(bi);
  wave_reduce2(best, bits, [&](float& v, float& ib, float w, float jb) {
    if (argmax_better(v, __float_as_int(ib), w, __float_as_int(jb))) {
      v = w;
      ib = jb;
    }
  });
  bi = __float_as_int(bits);
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kArgmaxThreads / 64; ++w)
      if (argmax_better(best, bi, sv[w], si[w])) {
        best = sv[w];
        bi = si[w];
      }
    const int tok = bi >= 0 && bi < V ? bi : 0;  // an all-NaN row falls back to token 0
    next_ids[b] = tok;
    out[(long long)b * out_stride + step] = tok;
  }
}

// One workgroup per row of full logits: strided scan, then the reduction.
__global__ __launch_bounds__(kArgmaxThreads) void argmax_rows_kernel(const float* __restrict__ logits, int V,
                                                                      int32_t* __restrict__ next_ids,
                                                                      int32_t* __restrict__ out, int out_stride,
                                                                      int step) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (long long)b * V;
  float best = -INFINITY;
  int bi = V;  // "none": loses every comparison below
  for (int n = tid; n < V; n += kArgmaxThreads) {
    const float v = row[n];
    if (v > best || (v == best && n < bi)) {
      best = v;
      bi = n;
    }
  }
  argmax_finish(best, bi, V, b, next_ids, out, out_stride, step);
}

// One workgroup per row of the head's (value, column) partials.
__global__ __launch_bounds__(kArgmaxThreads) void argmax_parts_kernel(const float2* __restrict__ part,
                                                                       int nparts, int V,
                                                                       int32_t* __restrict__ next_ids,
                                                                       int32_t* __restrict__ out, int out_stride,
                                                                       int step) {
  const int b = blockIdx.x, tid = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < nparts; i += kArgmaxThreads) {
    const float2 p = part[(long long)b * nparts + i];
    if (argmax_better(best, bi, p.x, __float_as_int(p.y))) {
      best = p.x;
      bi = __float_as_int(p.y);
    }
  }
  argmax_finish(best, bi, V, b, next_ids, out, out_stride, step);
}

void launch_argmax_rows(const float* logits, int B, int V, int32_t* next_ids, int32_t* out, int out_stride,
                        int step, hipStream_t s) {
  argmax_rows_kernel<<<B, kArgmaxThreads, 0, s>>>(logits, V, next_ids, out, out_stride, step);
}

void launch_argmax_parts(const void* part, int nparts, int B, int V, int32_t* next_ids, int32_t* out,
                         int out_stride, int step, hipStream_t s) {
  argmax_parts_kernel<<<B, kArgmaxThreads, 0, s>>>((const float2*)part, nparts, V, next_ids, out, out_stride,
                                                   step);
}

}  // namespace gpt2
