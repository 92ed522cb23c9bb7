// Bandwidth-bound variant over pre-materialised logits, and the loss.
//
// Same method as the fused path ("DPO Training on GPU, in depth", sections
// "What one DPO step computes" and "A training configuration that fits"), for
// a caller that already holds the [rows x T x V] logits the page's memory
// section sizes at 0.49 GiB per 2,048-token sequence in bf16.
//
//   k_stream_fwd   one workgroup per position (mask-0 ones only write zeros): a
//                  single pass over the V logits with a running (max, sum exp)
//                  per lane, 16-byte loads, then a fixed-order cross-lane
//                  combine -> lse, log p; k_stream_row_sums then sums each row
//   k_stream_bwd   dlogits = w (exp(x - lse) - onehot) rounded to bf16, exactly
//                  zero at positions outside the mask, in 16 KiB chunks
//   k_loss         the sigmoid DPO loss, its per-row gradient weights, rewards,
//                  margins and accuracy, in fp64 ("A worked example of the numbers"),
//                  with the reference-free, length-normalised and NLL-term variants
//   k_logits_mean  mean chosen / rejected logit from the forward's logit sums
// The streaming kernels take bf16 or fp32 logits (the page's memory section
// sizes fp32 logits of one 2,048-token sequence at 0.98 GiB).
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

// Element types of the logits: 16-byte vectors hold 8 bf16 or 4 fp32 values.
template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
  static __device__ __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(v[k]);
      x[2 * k + 1] = bf16_hi(v[k]);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float* d) {  // round to nearest even
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(d[2 * k], d[2 * k + 1]);
    return o;
  }
  static __device__ __forceinline__ float scalar(const void* base, size_t i) {
    return bf16_bits_to_float(((const uint16_t*)base)[i]);
  }
};
template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;
  static __device__ __forceinline__ void unpack(const u32x4 v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[k]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* d) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(d[k]);
    return o;
  }
  static __device__ __forceinline__ float scalar(const void* base, size_t i) {
    return ((const float*)base)[i];
  }
};

template <typename E>
__device__ __forceinline__ void absorb(float& m, float& s, const u32x4 v) {
  constexpr int N = Elem<E>::kPerVec;
  float x[N];
  Elem<E>::unpack(v, x);
  float lm = x[0];
#pragma unroll
  for (int k = 1; k < N; ++k) lm = fmaxf(lm, x[k]);
  if (lm > m) {
    s *= fast_exp2((m - lm) * kLog2e);  // 0 while m is still -inf (s is 0 then too)
    m = lm;
  }
  // while every value seen is -inf (logits masked out by the caller), m stays
  // -inf: a zero shift keeps exp2(-inf) = 0 instead of exp2(-inf + inf) = NaN
  const float ml = m == -INFINITY ? 0.f : m * kLog2e;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) acc += fast_exp2(fmaf(x[k], kLog2e, -ml));
  s += acc;
}

// One workgroup per position of [rows, T]: a mask-0 position only writes its
// zeros; a completion position reads its V logits once.  Per-position
// results stay at the position's flat index (no compaction pass: the row
// sums read the mask themselves), and a target outside [0, V) is recorded
// in a per-position flag that the row sums turn into the status word.
template <typename E>
__global__ __launch_bounds__(kStreamThreads) void k_stream_fwd(StreamFwdArgs a) {
  __shared__ float2 red[kStreamThreads / 64];
  const size_t pos = blockIdx.x;
  const int tid = threadIdx.x;
  if (pos == 0 && tid == 0) a.hdr->status = 0;  // the row sums run after this kernel and set it
  if (a.mask[pos] == 0) {
    if (tid == 0) {
      a.logp64[pos] = 0.0;
      a.bad[pos] = 0;
      if (a.lse_out) a.lse_out[pos] = 0.f;
    }
    return;
  }
  const u32x4* row = (const u32x4*)((const E*)a.logits + pos * a.V);
  const int nvec = a.V / Elem<E>::kPerVec;
  float mx = -INFINITY, s = 0.f;
  int v = tid;
  for (; v + (kStreamUnroll - 1) * kStreamThreads < nvec; v += kStreamUnroll * kStreamThreads) {
    u32x4 buf[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) buf[u] = __builtin_nontemporal_load(row + v + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) absorb<E>(mx, s, buf[u]);
  }
  for (; v < nvec; v += kStreamThreads) absorb<E>(mx, s, __builtin_nontemporal_load(row + v));
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
    const int t = a.targets[pos];
    const bool ok = t >= 0 && t < a.V;
    a.logp64[pos] = ok ? (double)Elem<E>::scalar(a.logits, pos * a.V + t) - lse : __builtin_nan("");
    a.bad[pos] = ok ? 0 : 1;
    if (a.lse_out) a.lse_out[pos] = (float)lse;
  }
}

// Row sums over the flat per-position log p of the streaming forward, in a
// fixed order (each thread a strided share of the row, then a tree), with
// the row's completion count; a row holding an out-of-range target sets the
// status word (reset by the forward kernel, which ran before).
__global__ __launch_bounds__(256) void k_stream_row_sums(StreamRowSumArgs a) {
  __shared__ double red[256];
  __shared__ int cnt[256];
  __shared__ int flag[256];
  const int r = blockIdx.x;
  const size_t base = (size_t)r * a.T;
  double s = 0.0;
  int c = 0, f = 0;
  for (int t = threadIdx.x; t < a.T; t += 256) {
    const bool on = a.mask[base + t] != 0;
    s += on ? a.logp64[base + t] : 0.0;
    c += on;
    f |= on ? a.bad[base + t] : 0;
  }
  red[threadIdx.x] = s;
  cnt[threadIdx.x] = c;
  flag[threadIdx.x] = f;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      red[threadIdx.x] += red[threadIdx.x + o];
      cnt[threadIdx.x] += cnt[threadIdx.x + o];
      flag[threadIdx.x] |= flag[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double v = red[0];
    if (a.sum32) a.sum32[r] = (float)v;
    if (a.sum64) a.sum64[r] = v;
    if (a.n_tokens) a.n_tokens[r] = cnt[0];
    if (flag[0]) atomicOr(&a.hdr->status, kStatusTargetRange);
  }
}

// The backward walks [positions x V] in 16 KiB chunks (four 16-byte vectors
// per thread), consecutive workgroups on consecutive chunks: the chunks in
// flight at any moment form one contiguous stretch of the logits and of
// dlogits, which this part reads and writes back ~8 % faster than one
// workgroup per 256 KiB row (the rows' streams then sit 256 KiB apart).
constexpr int kBwdVecs = 4;
constexpr int kBwdChunk = kBwdVecs * kStreamThreads;  // 16-byte vectors per chunk

template <typename E>
__global__ __launch_bounds__(kStreamThreads) void k_stream_bwd(StreamBwdArgs a, long positions) {
  constexpr int N = Elem<E>::kPerVec;
  const int tid = threadIdx.x;
  const int nvec = a.V / N;
  const int cpr = (nvec + kBwdChunk - 1) / kBwdChunk;  // chunks per row
  const long total = positions * cpr;
  for (long c = blockIdx.x; c < total; c += gridDim.x) {
    const long p = c / cpr;
    const int v0 = (int)(c - p * cpr) * kBwdChunk;
    u32x4* out = (u32x4*)((E*)a.d_logits + p * a.V);
    // the position's four scalars in one go (all valid at every position), so
    // a completion chunk waits for one load latency before its row loads
    const uint8_t mk = a.mask[p];
    int tg = a.targets[p];
    const float lse = a.lse[p];
    const float w = a.weight[p / a.T];
    if (mk == 0) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kBwdVecs; ++u) {
        const int v = v0 + u * kStreamThreads + tid;
        if (v < nvec) __builtin_nontemporal_store(z, out + v);
      }
      continue;
    }
    if (tg < 0 || tg >= a.V) {
      if (tid == 0 && v0 == 0) atomicOr(&a.hdr->status, kStatusTargetRange);
      tg = -1;
    }
    const float L = lse * kLog2e;
    const int tv = tg >= 0 ? tg / N : -1;  // the one vector holding the target
    const u32x4* row = (const u32x4*)((const E*)a.logits + p * a.V);
    u32x4 buf[kBwdVecs];
#pragma unroll
    for (int u = 0; u < kBwdVecs; ++u) {
      const int v = v0 + u * kStreamThreads + tid;
      if (v < nvec) buf[u] = __builtin_nontemporal_load(row + v);
    }
#pragma unroll
    for (int u = 0; u < kBwdVecs; ++u) {
      const int v = v0 + u * kStreamThreads + tid;
      if (v >= nvec) break;
      float x[N], d[N];
      Elem<E>::unpack(buf[u], x);
#pragma unroll
      for (int k = 0; k < N; ++k) d[k] = w * fast_exp2(fmaf(x[k], kLog2e, -L));
      if (v == tv) {
#pragma unroll
        for (int k = 0; k < N; ++k) d[k] = (k == tg % N) ? d[k] - w : d[k];
      }
      __builtin_nontemporal_store(Elem<E>::pack(d), out + v);
    }
  }
}

__global__ void k_reset_status(WsHeader* hdr) { hdr->status = 0; }

// the call's status for a caller without a workspace: `code` if a target was
// out of range, else 0
__global__ void k_write_status(const WsHeader* hdr, int code, int32_t* out) {
  out[0] = (hdr->status & kStatusTargetRange) ? code : 0;
}

// ---------------------------------------------------------------------------
// sigmoid DPO loss, fp64
// ---------------------------------------------------------------------------
__device__ __forceinline__ double softplus_d(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
__device__ __forceinline__ double sigmoid_d(double x) {
  const double e = exp(-fabs(x));
  return x >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

// Variants on the same scores: a NULL reference means reference-free scores;
// length_norm divides each row's policy and reference score by its completion
// token count (a row without tokens averages to 0); alpha > 0 adds alpha
// times the mean negative log-probability per chosen completion token of the
// batch (-sum pi_chosen / sum n_chosen) to the loss.
__global__ __launch_bounds__(256) void k_loss(LossArgs a) {
  __shared__ double red_l[256];
  __shared__ long long red_n[256];
  __shared__ int red_c[256];
  const int tid = threadIdx.x;
  const int B = a.num_pairs;
  auto chosen = [&](int i) { return a.layout == 0 ? 2 * i : i; };
  auto rejected = [&](int i) { return a.layout == 0 ? 2 * i + 1 : B + i; };
  // chosen-row totals for the NLL term, in a fixed order
  double nll = 0.0, inv_nch = 0.0;
  if (a.n_tokens) {
    double ps = 0.0;
    long long nc = 0;
    for (int i = tid; i < B; i += 256) {
      ps += a.policy[chosen(i)];
      nc += a.n_tokens[chosen(i)];
    }
    red_l[tid] = ps;
    red_n[tid] = nc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        red_l[tid] += red_l[tid + o];
        red_n[tid] += red_n[tid + o];
      }
      __syncthreads();
    }
    if (red_n[0] > 0) {
      nll = -red_l[0] / (double)red_n[0];
      inv_nch = 1.0 / (double)red_n[0];
    }
    __syncthreads();
  }
  auto scale = [&](int r) {
    if (!a.length_norm) return 1.0;
    const int n = a.n_tokens[r];
    return n > 0 ? 1.0 / (double)n : 0.0;
  };
  double lsum = 0.0;
  int correct = 0;
  for (int i = tid; i < B; i += 256) {
    const int rc = chosen(i), rr = rejected(i);
    const double sc = scale(rc), sr = scale(rr);
    const double ref_c = a.ref ? (double)a.ref[rc] : 0.0;
    const double ref_r = a.ref ? (double)a.ref[rr] : 0.0;
    const double reward_c = a.beta * (a.policy[rc] - ref_c) * sc;
    const double reward_r = a.beta * (a.policy[rr] - ref_r) * sr;
    const double margin = reward_c - reward_r;
    lsum += softplus_d(-margin);
    correct += margin > 0.0;
    const double g = a.beta * sigmoid_d(-margin) / (double)B;
    a.weight[rc] = (float)(g * sc + a.alpha * inv_nch);
    a.weight[rr] = (float)(-g * sr);
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
    a.loss[0] = (float)(red_l[0] / (double)B + a.alpha * nll);
    if (a.accuracy) a.accuracy[0] = (float)((double)red_c[0] / (double)B);
    if (a.nll) a.nll[0] = (float)nll;
  }
}

// mean logit over completion positions and vocabulary, chosen and rejected halves
__global__ __launch_bounds__(256) void k_logits_mean(LogitsMeanArgs a) {
  __shared__ double red_s[2][256];
  __shared__ long long red_n[2][256];
  const int tid = threadIdx.x;
  const int B = a.num_pairs;
  double s0 = 0.0, s1 = 0.0;
  long long n0 = 0, n1 = 0;
  for (int i = tid; i < B; i += 256) {
    const int rc = a.layout == 0 ? 2 * i : i;
    const int rr = a.layout == 0 ? 2 * i + 1 : B + i;
    s0 += a.logit_sum[rc];
    n0 += a.n_tokens[rc];
    s1 += a.logit_sum[rr];
    n1 += a.n_tokens[rr];
  }
  red_s[0][tid] = s0;
  red_s[1][tid] = s1;
  red_n[0][tid] = n0;
  red_n[1][tid] = n1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      for (int h = 0; h < 2; ++h) {
        red_s[h][tid] += red_s[h][tid + o];
        red_n[h][tid] += red_n[h][tid + o];
      }
    }
    __syncthreads();
  }
  if (tid < 2) {
    const long long n = red_n[tid][0];
    a.means[tid] = n > 0 ? (float)(red_s[tid][0] / ((double)n * (double)a.V)) : 0.f;
  }
}

hipError_t launch_stream_fwd(const StreamFwdArgs& a, long positions, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_fwd<uint16_t>, dim3((unsigned)positions), dim3(kStreamThreads), 0, s, a);
  return hipGetLastError();
}

// grid: workgroups in flight (a multiple of the CU count); they stride over the chunks
static unsigned bwd_grid(const StreamBwdArgs& a, long positions, int elems_per_vec, int grid) {
  const long cpr = (a.V / elems_per_vec + kBwdChunk - 1) / kBwdChunk;
  return (unsigned)std::max(1L, std::min<long>(positions * cpr, grid));
}

hipError_t launch_stream_bwd(const StreamBwdArgs& a, long positions, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_bwd<uint16_t>, dim3(bwd_grid(a, positions, 8, grid)), dim3(kStreamThreads), 0, s, a,
                     positions);
  return hipGetLastError();
}

hipError_t launch_stream_fwd_f32(const StreamFwdArgs& a, long positions, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_fwd<float>, dim3((unsigned)positions), dim3(kStreamThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_bwd_f32(const StreamBwdArgs& a, long positions, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_bwd<float>, dim3(bwd_grid(a, positions, 4, grid)), dim3(kStreamThreads), 0, s, a,
                     positions);
  return hipGetLastError();
}

hipError_t launch_stream_row_sums(const StreamRowSumArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_row_sums, dim3(a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_logits_mean(const LogitsMeanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_logits_mean, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_write_status(const WsHeader* hdr, int code, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_write_status, dim3(1), dim3(1), 0, s, hdr, code, out);
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
