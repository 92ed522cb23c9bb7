// Bandwidth-bound variant over pre-materialised bf16 logits, and the loss.
//
// Same method as the fused path ("DPO Training on GPU, in depth", sections
// "What one DPO step computes" and "A training configuration that fits"), for
// a caller that already holds the [rows x T x V] logits the page's memory
// section sizes at 0.49 GiB per 2,048-token sequence in bf16.
//
//   k_stream_fwd   one workgroup per completion position: a single pass over
//                  the V logits with a running (max, sum exp) per lane, 16-byte
//                  loads, then a fixed-order cross-lane combine -> lse, log p
//   k_stream_bwd   one workgroup per position: dlogits = w (exp(x - lse) - onehot)
//                  rounded to bf16, exactly zero at positions outside the mask
//   k_loss         the sigmoid DPO loss, its per-row gradient weights, rewards,
//                  margins and accuracy, in fp64 ("A worked example of the numbers")
#include "dpo_common.h"
#include "launch.h"

namespace dpo {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

// merge running (max, sum) pairs: sum is relative to max
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  // an empty partial is (-inf, 0) and contributes nothing
  const float M = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.f : s * fast_exp2((m - M) * kLog2e);
  const float b = m2 == -INFINITY ? 0.f : s2 * fast_exp2((m2 - M) * kLog2e);
  s = a + b;
  m = M;
}

__device__ __forceinline__ void absorb8(float& m, float& s, const u32x4 v) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_lo(v[k]);
    x[2 * k + 1] = bf16_hi(v[k]);
  }
  float lm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  if (lm > m) {
    s *= fast_exp2((m - lm) * kLog2e);
    m = lm;
  }
  const float ml = m * kLog2e;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc += fast_exp2(fmaf(x[k], kLog2e, -ml));
  s += acc;
}

__global__ __launch_bounds__(kStreamThreads) void k_stream_fwd(StreamFwdArgs a) {
  __shared__ float2 red[kStreamThreads / 64];
  const int m = blockIdx.x;
  if (m >= a.hdr->n_c) return;
  const int tid = threadIdx.x;
  const size_t pos = (size_t)a.idx[m];
  const u32x4* row = (const u32x4*)(a.logits + pos * a.V);
  const int nvec = a.V / 8;
  float mx = -INFINITY, s = 0.f;
  int v = tid;
  for (; v + (kStreamUnroll - 1) * kStreamThreads < nvec; v += kStreamUnroll * kStreamThreads) {
    u32x4 buf[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) buf[u] = __builtin_nontemporal_load(row + v + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) absorb8(mx, s, buf[u]);
  }
  for (; v < nvec; v += kStreamThreads) absorb8(mx, s, __builtin_nontemporal_load(row + v));
  // fixed-order combine: wave butterflies, then the 4 waves in order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    lse_merge(mx, s, m2, s2);
  }
  if ((tid & 63) == 0) red[tid >> 6] = make_float2(mx, s);
  __syncthreads();
  if (tid == 0) {
    float M = red[0].x, S = red[0].y;
    for (int w = 1; w < kStreamThreads / 64; ++w) lse_merge(M, S, red[w].x, red[w].y);
    const double lse = (double)M + log((double)S);
    const int t = a.tgt_c[m];
    a.lse64[m] = lse;
    a.logp64[m] = t >= 0 ? (double)bf16_bits_to_float(a.logits[pos * a.V + t]) - lse : __builtin_nan("");
    if (a.lse_out) a.lse_out[pos] = (float)lse;
  }
}

constexpr int kBwdUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void k_stream_bwd(StreamBwdArgs a) {
  const size_t p = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = a.V / 8;
  u32x4* out = (u32x4*)(a.d_logits + p * a.V);
  if (a.mask[p] == 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int v = tid; v < nvec; v += kStreamThreads) __builtin_nontemporal_store(z, out + v);
    return;
  }
  int tg = a.targets[p];
  if (tg < 0 || tg >= a.V) {
    if (tid == 0) atomicOr(&a.hdr->status, kStatusTargetRange);
    tg = -1;
  }
  const float L = a.lse[p] * kLog2e;
  const float w = a.weight[p / a.T];
  const int tv = tg >= 0 ? tg >> 3 : -1;  // the one vector holding the target
  const u32x4* row = (const u32x4*)(a.logits + p * a.V);
  for (int v0 = tid; v0 < nvec; v0 += kBwdUnroll * kStreamThreads) {
    u32x4 buf[kBwdUnroll];
#pragma unroll
    for (int u = 0; u < kBwdUnroll; ++u) {
      const int v = v0 + u * kStreamThreads;
      if (v < nvec) buf[u] = __builtin_nontemporal_load(row + v);
    }
#pragma unroll
    for (int u = 0; u < kBwdUnroll; ++u) {
      const int v = v0 + u * kStreamThreads;
      if (v >= nvec) break;
      float d[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        d[2 * k] = w * fast_exp2(fmaf(bf16_lo(buf[u][k]), kLog2e, -L));
        d[2 * k + 1] = w * fast_exp2(fmaf(bf16_hi(buf[u][k]), kLog2e, -L));
      }
      if (v == tv) {
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = (k == (tg & 7)) ? d[k] - w : d[k];
      }
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(d[2 * k], d[2 * k + 1]);
      __builtin_nontemporal_store(o, out + v);
    }
  }
}

__global__ void k_reset_status(WsHeader* hdr) { hdr->status = 0; }

// ---------------------------------------------------------------------------
// sigmoid DPO loss, fp64
// ---------------------------------------------------------------------------
__device__ __forceinline__ double softplus_d(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
__device__ __forceinline__ double sigmoid_d(double x) {
  const double e = exp(-fabs(x));
  return x >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

__global__ __launch_bounds__(256) void k_loss(LossArgs a) {
  __shared__ double red_l[256];
  __shared__ int red_c[256];
  const int tid = threadIdx.x;
  const int B = a.num_pairs;
  double lsum = 0.0;
  int correct = 0;
  for (int i = tid; i < B; i += 256) {
    const int rc = a.layout == 0 ? 2 * i : i;
    const int rr = a.layout == 0 ? 2 * i + 1 : B + i;
    const double reward_c = a.beta * (a.policy[rc] - (double)a.ref[rc]);
    const double reward_r = a.beta * (a.policy[rr] - (double)a.ref[rr]);
    const double margin = reward_c - reward_r;
    lsum += softplus_d(-margin);
    correct += margin > 0.0;
    const double g = a.beta * sigmoid_d(-margin) / (double)B;
    a.weight[rc] = (float)g;
    a.weight[rr] = (float)(-g);
    if (a.reward) {
      a.reward[rc] = (float)reward_c;
      a.reward[rr] = (float)reward_r;
    }
    if (a.margin) a.margin[i] = (float)margin;
  }
  red_l[tid] = lsum;
  red_c[tid] = correct;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      red_l[tid] += red_l[tid + o];
      red_c[tid] += red_c[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.loss[0] = (float)(red_l[0] / (double)B);
    if (a.accuracy) a.accuracy[0] = (float)((double)red_c[0] / (double)B);
  }
}

hipError_t launch_stream_fwd(const StreamFwdArgs& a, long positions, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_fwd, dim3((unsigned)positions), dim3(kStreamThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_bwd(const StreamBwdArgs& a, long positions, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_bwd, dim3((unsigned)positions), dim3(kStreamThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reset_status(WsHeader* hdr, hipStream_t s) {
  hipLaunchKernelGGL(k_reset_status, dim3(1), dim3(1), 0, s, hdr);
  return hipGetLastError();
}

hipError_t launch_loss(const LossArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_loss, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dpo
