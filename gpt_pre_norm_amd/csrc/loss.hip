// Next-token cross-entropy of the tied head's logits: loss = log sum_n
// exp(logit_n) - logit_target per row ("Full Forward Pass", How it works:
// callers take the logits and a next-token cross-entropy), with the
// log-sum-exp taken about the row maximum.
#include "kernels.h"

namespace gpt2 {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

GPT2_DEV void merge(float& m, float& s, float m2, float s2) {
  // combine two (max, sum of exp(x - max)) states; an empty state has s = 0
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
  m = mn;
}

GPT2_DEV float finish(float m, float s, float t, int target, int N, uint32_t* flags) {
  if (target < 0 || target >= N) {
    atomicOr(flags, 1u);
    return __builtin_nanf("");
  }
  return m + __builtin_amdgcn_logf(s) * kLn2 - t;
}
}  // namespace

// one wave per row: the partial states of the row's column tiles
__global__ __launch_bounds__(64) void loss_parts_kernel(const float2* __restrict__ part, int nparts,
                                                        const float* __restrict__ tgt,
                                                        const int32_t* __restrict__ targets, int N,
                                                        float* __restrict__ loss, uint32_t* flags) {
  const int m = blockIdx.x, lane = threadIdx.x;
  float mx = -INFINITY, sm = 0.f;
  for (int i = lane; i < nparts; i += 64) {
    const float2 p = part[(long long)m * nparts + i];
    merge(mx, sm, p.x, p.y);
  }
  wave_reduce2(mx, sm, merge);
  if (lane == 0) {
    const int t = targets[m];
    loss[m] = finish(mx, sm, t >= 0 && t < N ? tgt[m] : 0.f, t, N, flags);
  }
}

// one workgroup per row of full logits
__global__ __launch_bounds__(256) void loss_logits_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ targets, int N,
                                                          float* __restrict__ loss, uint32_t* flags) {
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = logits + (long long)m * N;
  float mx = -INFINITY, sm = 0.f;
  for (int n = tid; n < N; n += 256) merge(mx, sm, row[n], 1.f);
  wave_reduce2(mx, sm, merge);
  __shared__ float wm[4], ws[4];
  if (lane == 0) {
    wm[wave] = mx;
    ws[wave] = sm;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) merge(mx, sm, wm[w], ws[w]);
    const int t = targets[m];
    loss[m] = finish(mx, sm, t >= 0 && t < N ? row[t] : 0.f, t, N, flags);
  }
}

void launch_loss_from_parts(const void* part, int nparts, const float* tgt, const int32_t* targets, int M,
                            int N, float* loss, uint32_t* flags, hipStream_t s) {
  loss_parts_kernel<<<M, 64, 0, s>>>((const float2*)part, nparts, tgt, targets, N, loss, flags);
}

void launch_loss_from_logits(const float* logits, const int32_t* targets, int M, int N, float* loss,
                             uint32_t* flags, hipStream_t s) {
  loss_logits_kernel<<<M, 256, 0, s>>>(logits, targets, N, loss, flags);
}

}  // namespace gpt2
