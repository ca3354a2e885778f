// ep_row_kernels.h -- the row kernels: dispatch scatter (bf16 rows, or per-token
// dynamic fp8 / int8 codes, optionally after per-expert smoothing), the
// weighted combine gather (of bf16 or quantised rows, optionally fused with
// the residual add and RMSNorm), and the 1-D uneven all-to-all (plan + chunk
// copy).
//
// Token-major: a token's positions (K <= 16) are read once by the first K
// lanes of a wavefront and broadcast with v_readlane, so the row loops carry
// no per-element index math; every row moves as 16-byte vectors, 64 lanes
// side by side (1 KiB per wave instruction), fully coalesced.
#pragma once

#include "ep_common.h"

namespace ep {

constexpr int kRowThreads = 256;                       // 4 waves
constexpr int kTokensPerBlock = kRowThreads / kWave;   // one token per wave

// Cache policy of the row streams: non-temporal (streaming) or default.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4* p, const u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Lane k < K of a token's wave reads pos[t][k]; a row outside [0, cap_rows)
// other than -1 is a caller error: it is dropped and flagged, never followed.
__device__ __forceinline__ int row_of(const int32_t* __restrict__ pos, int t, int K, int lane,
                                      int64_t cap_rows) {
  if (lane >= K) return -1;
  const int p = pos[(int64_t)t * K + lane];
  if (p >= 0 && (int64_t)p >= cap_rows) {
    raise_device_error(kErrBadRow);
    return -1;
  }
  return p < 0 ? -1 : p;
}

// ---------------------------------------------------------------------------
// Dispatch, bf16 rows: expand_x[pos[t][k]] = x[t] for every live copy
// (_allToAllV_2d_index_push_kernel on the PyTorch compare view
// "ciflow/h100-symm-mem/166772" puts one row per (token, k)).
// Work item: one wavefront per (token, column chunk of 64*U vectors), so a
// launch holds T * ceil(V / 64U) small items and the last wave of items is
// short (one wave per whole token leaves a long tail at these T).  x is read
// once per item, each chunk is written to the K rows.
// ---------------------------------------------------------------------------
template <int U, bool NTL, bool NTS>
__global__ __launch_bounds__(kRowThreads) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ ex,
    const float* __restrict__ weights, float* __restrict__ expand_weights, int T, int K, int V,
    int chunks, int64_t cap_rows) {
  const int64_t g = (int64_t)blockIdx.x * kTokensPerBlock + uniform((int)(threadIdx.x / kWave));
  const int64_t t64 = g / chunks;
  if (t64 >= T) return;
  const int t = (int)t64;
  const int v0 = (int)(g - t64 * chunks) * kWave * U;
  const int lane = lane_id();
  const int my_pos = row_of(pos, t, K, lane, cap_rows);
  const uint64_t live = ballot(my_pos >= 0);
  if (live == 0) return;  // inactive token: x is not read
  if (v0 == 0 && expand_weights != nullptr && my_pos >= 0)
    expand_weights[my_pos] = weights[(int64_t)t * K + lane];
  const u32x4* src = x + (int64_t)t * V;
  u32x4 r[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = v0 + u * kWave + lane;
    if (idx < V) r[u] = ld<NTL>(src + idx);
  }
  uint64_t m = live;
  while (m) {
    const int k = __builtin_ctzll(m);
    m &= m - 1;
    const int p = __builtin_amdgcn_readlane(my_pos, k);
    u32x4* dst = ex + (int64_t)p * V;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = v0 + u * kWave + lane;
      if (idx < V) st<NTS>(dst + idx, r[u]);
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch with per-token dynamic quantisation (quantMode 2 of the CANN
// "aclnnMoeDistributeDispatchV2" page; one fp32 scale per expanded row, as
// dynamicScalesOut), to OCP fp8 E4M3FN or int8:
//   scale = fl32(amax / qmax),  code = encode(fl32(x / scale)),
// qmax = 448 (E4M3FN, round to nearest even, saturating) or 127 (int8,
// nearest integer, ties to even, clamped).
// ---------------------------------------------------------------------------

// fp32 -> E4M3FN, round to nearest even, saturating to +-448; NaN -> 0x7f.
__device__ __forceinline__ uint32_t e4m3fn_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t mag;
  if (a > 0x7f800000u) {
    mag = 0x7fu;
  } else if (a >= 0x43e00000u) {  // |v| >= 448 (infinity included): saturate
    mag = 0x7eu;
  } else if (a >= 0x3c800000u) {  // 2^-6 <= |v| < 448: normal codes
    const uint32_t q = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
    const uint32_t rest = a & 0xfffffu;
    mag = q + ((rest > 0x80000u) | ((rest == 0x80000u) & (q & 1u)));
  } else {  // subnormal codes are the multiples of 2^-9 below 2^-6
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return sign | mag;
}

// int8 code: nearest integer, ties to even (v_rndne), clamped to +-127.
__device__ __forceinline__ uint32_t int8_code(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)((int32_t)r) & 0xffu;
}

constexpr int kQFp8 = 1;
constexpr int kQInt8 = 2;

template <int QT>
__device__ __forceinline__ uint32_t quant_code(float v) {
  if constexpr (QT == kQFp8) return e4m3fn_code(v);
  else return int8_code(v);
}

template <int QT>
__device__ __forceinline__ float quant_max() {
  if constexpr (QT == kQFp8) return 448.0f;
  else return 127.0f;
}

// Quantise 16 fp32 values into 16 codes (zero codes when scale == 0).
template <int QT>
__device__ __forceinline__ u32x4 quantize16f(const float* f, float scale) {
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c[4] = {0, 0, 0, 0};
    if (scale != 0.0f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = quant_code<QT>(f[4 * i + j] / scale);
    }
    out[i] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  }
  return u32x4{out[0], out[1], out[2], out[3]};
}

// x / scale for one row's scale, correctly rounded, from values prepared
// once per row.  r is the correctly rounded 1/s: one Newton step
// r0 + r0 (1 - s r0) from v_rcp_f32's result (specified to 1 ulp) gives it
// for every scale except those whose mantissa is all ones, s = 2^k (2 -
// 2^-23); there 1/s = 2^-k-1 (1 + 2^-24 + 2^-48 + ...), just above the
// midpoint of 2^-k-1 and its successor, and the step can stop on the
// midpoint and round down, so r is set to that successor directly.  Then
// rd + rl is 1/s to about 2^-48: rd is r or the float below it, whichever
// is not above 1/s, and rl = (1 - s rd) rd >= 0.  Per element,
//   q0 = fma(n, rd, n rl)        within half an ulp and a little of n/s,
//   q  = q0 - (s q0 - n) r       (two fused multiply-adds),
// and q is the correctly rounded n/s (Markstein's theorem: the remainder of
// a faithful quotient is exact, and one correction with the correctly
// rounded reciprocal rounds correctly).  rl >= 0 keeps the sign of a zero n
// through q0, and the remainder is formed negated (s q - n) and subtracted so
// that a -0 stays -0.  (Checked on the host over every mantissa, and for the
// quotients on and around every code's rounding boundaries.)  The fast form
// is taken for scales in [2^-60, 2^60]; there every quotient of at least
// 2^-11 in magnitude has normal operands and an exact remainder, and smaller
// quotients give codes of zero.  Other scales (zero, subnormal, huge,
// infinite, NaN) take the plain division.
struct RowDiv {
  float s, r, rd, rl;
  bool fast;
};

__device__ __forceinline__ RowDiv row_div(float scale) {
  RowDiv d;
  d.s = __int_as_float(uniform(__float_as_int(scale)));
  d.fast = d.s >= 0x1p-60f && d.s <= 0x1p60f;
  const float r0 = __builtin_amdgcn_rcpf(d.s);
  d.r = __builtin_fmaf(__builtin_fmaf(-d.s, r0, 1.0f), r0, r0);
  const uint32_t sb = __float_as_uint(d.s);
  if ((sb & 0x7fffffu) == 0x7fffffu)  // all-ones mantissa: 1/s rounds to 2^-k-1 (1 + 2^-23)
    d.r = __uint_as_float(((253u - ((sb >> 23) & 0xffu)) << 23) | 1u);
  d.rd = __builtin_fmaf(-d.s, d.r, 1.0f) < 0.0f ? __uint_as_float(__float_as_uint(d.r) - 1u) : d.r;
  d.rl = __builtin_fmaf(-d.s, d.rd, 1.0f) * d.rd;
  return d;
}

__device__ __forceinline__ float div_fast(float n, const RowDiv& d) {
  const float q0 = __builtin_fmaf(n, d.rd, n * d.rl);
  const float e = __builtin_fmaf(d.s, q0, -n);
  return __builtin_fmaf(-e, d.r, q0);
}

// Fast-path codes of 16 quotients.  fp8: gfx950's v_cvt_pk_fp8_f32 rounds
// to nearest even into OCP E4M3FN and, after a clamp to +-448 (v_med3),
// gives the code e4m3fn_code gives for every non-NaN input (all 2^32 fp32
// patterns compared); the fast path never sees NaN.  int8: v_rndne, clamp,
// convert.
template <int QT>
__device__ __forceinline__ u32x4 quantize16_fast(const float* f, const RowDiv& d) {
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = div_fast(f[4 * i + j], d);
    if constexpr (QT == kQFp8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = __builtin_amdgcn_fmed3f(v[j], -448.0f, 448.0f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
      out[i] = (uint32_t)w;
    } else {
      out[i] = int8_code(v[0]) | (int8_code(v[1]) << 8) | (int8_code(v[2]) << 16) | (int8_code(v[3]) << 24);
    }
  }
  return u32x4{out[0], out[1], out[2], out[3]};
}

// Codes of 16 values of one row: the fast path, or the plain division and
// the software encoders for rows whose scale is outside its range (a
// row-uniform branch).
template <int QT>
__device__ __forceinline__ u32x4 quantize16r(const float* f, const RowDiv& d) {
  if (d.fast) return quantize16_fast<QT>(f, d);
  return quantize16f<QT>(f, d.s);
}

__device__ __forceinline__ void unpack16(const u32x4 a, const u32x4 b, float* f) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = bf16lo(w[i]);
    f[2 * i + 1] = bf16hi(w[i]);
  }
}

// Quantise 16 bf16 values (two 16-byte vectors) into 16 codes.
template <int QT>
__device__ __forceinline__ u32x4 quantize16(const u32x4 a, const u32x4 b, const RowDiv& d) {
  float f[16];
  unpack16(a, b, f);
  return quantize16r<QT>(f, d);
}

// Largest bf16 magnitude of two vectors, as the 15-bit magnitude pattern
// (non-negative floats order like their bit patterns).
__device__ __forceinline__ uint32_t amax16_bits(const u32x4 a, const u32x4 b, uint32_t m) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = max(m, w[i] & 0x7fffu);
    m = max(m, (w[i] >> 16) & 0x7fffu);
  }
  return m;
}

// One workgroup (4 waves) per token: thread i owns the 16-value groups
// i, i + 256, ...; the first G of them stay in VGPRs between the amax pass and
// the quantise pass, longer rows re-read the rest.  The row's amax is
// reduced across lanes with shuffles and across the 4 waves through LDS.
template <int QT, int G, bool NTL, bool NTS>
__global__ __launch_bounds__(kRowThreads) void dispatch_quant_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ q,
    float* __restrict__ scales, const float* __restrict__ weights,
    float* __restrict__ expand_weights, int T, int K, int NG, int64_t cap_rows) {
  __shared__ uint32_t s_max[kRowThreads / kWave];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int my_pos = row_of(pos, t, K, lane, cap_rows);
  const uint64_t live = ballot(my_pos >= 0);  // the same in every wave of the token
  if (live == 0) return;
  const u32x4* src = x + (int64_t)t * NG * 2;

  u32x4 cache[G][2];
  uint32_t mbits = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = g * kRowThreads + tid;
    if (idx < NG) {
      cache[g][0] = ld<NTL>(src + 2 * idx);
      cache[g][1] = ld<NTL>(src + 2 * idx + 1);
      mbits = amax16_bits(cache[g][0], cache[g][1], mbits);
    }
  }
  for (int idx = G * kRowThreads + tid; idx < NG; idx += kRowThreads)
    mbits = amax16_bits(ld<NTL>(src + 2 * idx), ld<NTL>(src + 2 * idx + 1), mbits);
  mbits = wave_max_u32(mbits);
  if (lane == 0) s_max[wave] = mbits;
  __syncthreads();
  uint32_t m = s_max[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / kWave; ++w) m = max(m, s_max[w]);
  const float amax = __uint_as_float(m << 16);
  const float scale = amax / quant_max<QT>();
  const RowDiv rd = row_div(scale);

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = g * kRowThreads + tid;
    if (idx < NG) {
      const u32x4 code = quantize16<QT>(cache[g][0], cache[g][1], rd);
      uint64_t mk = live;
      while (mk) {
        const int k = __builtin_ctzll(mk);
        mk &= mk - 1;
        const int p = __builtin_amdgcn_readlane(my_pos, k);
        st<NTS>(q + (int64_t)p * NG + idx, code);
      }
    }
  }
  for (int idx = G * kRowThreads + tid; idx < NG; idx += kRowThreads) {
    const u32x4 code = quantize16<QT>(ld<NTL>(src + 2 * idx), ld<NTL>(src + 2 * idx + 1), rd);
    uint64_t mk = live;
    while (mk) {
      const int k = __builtin_ctzll(mk);
      mk &= mk - 1;
      const int p = __builtin_amdgcn_readlane(my_pos, k);
      st<NTS>(q + (int64_t)p * NG + idx, code);
    }
  }
  if (wave == 0 && my_pos >= 0) {
    scales[my_pos] = scale;
    if (expand_weights != nullptr) expand_weights[my_pos] = weights[(int64_t)t * K + lane];
  }
}

// ---------------------------------------------------------------------------
// Weighted combine: out[t] = bf16_rne(sum_k w[t][k] * y[pos[t][k]]), fp32
// fused multiply-adds in increasing k from +0; copies with pos < 0 add
// nothing.  Work item: one wavefront per (token, column chunk of 64*U
// vectors); all K row chunks are loaded before the first FMA so the K
// gathers are in flight together.
// ---------------------------------------------------------------------------
template <int KMAX, int U, int WPB, bool NTL, bool NTS>
__global__ __launch_bounds__(WPB * kWave) void combine_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pos,
    const float* __restrict__ w, u32x4* __restrict__ out, int T, int K, int V, int chunks,
    int64_t cap_rows) {
  const int64_t g = (int64_t)blockIdx.x * WPB + uniform((int)(threadIdx.x / kWave));
  const int64_t t64 = g / chunks;
  if (t64 >= T) return;
  const int t = (int)t64;
  const int v0 = (int)(g - t64 * chunks) * kWave * U;
  const int lane = lane_id();
  const int my_pos = row_of(pos, t, K, lane, cap_rows);
  const float my_w = lane < K ? w[(int64_t)t * K + lane] : 0.0f;
  int pk[KMAX];
  float wk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    pk[k] = __builtin_amdgcn_readlane(my_pos, k);
    wk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k));
  }
  u32x4 r[KMAX][U];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (pk[k] >= 0) {
      const u32x4* row = y + (int64_t)pk[k] * V;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = v0 + u * kWave + lane;
        if (idx < V) r[k][u] = ld<NTL>(row + idx);
      }
    }
  }
  float acc[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (pk[k] >= 0) {
      const float wt = wk[k];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t v4[4] = {r[k][u].x, r[k][u].y, r[k][u].z, r[k][u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[u][2 * i] = __builtin_fmaf(wt, bf16lo(v4[i]), acc[u][2 * i]);
          acc[u][2 * i + 1] = __builtin_fmaf(wt, bf16hi(v4[i]), acc[u][2 * i + 1]);
        }
      }
    }
  }
  u32x4* dst = out + (int64_t)t * V;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = v0 + u * kWave + lane;
    if (idx < V) {
      u32x4 o;
      o.x = f32_to_bf16_rne(acc[u][0]) | (f32_to_bf16_rne(acc[u][1]) << 16);
      o.y = f32_to_bf16_rne(acc[u][2]) | (f32_to_bf16_rne(acc[u][3]) << 16);
      o.z = f32_to_bf16_rne(acc[u][4]) | (f32_to_bf16_rne(acc[u][5]) << 16);
      o.w = f32_to_bf16_rne(acc[u][6]) | (f32_to_bf16_rne(acc[u][7]) << 16);
      st<NTS>(dst + idx, o);
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch with per-expert smoothing before per-copy dynamic quantisation
// (scalesOptional of shape (E, H) with quantMode 2 on the CANN dispatch
// page): for every live copy (t, k) of expert e, xs = fl32(x[t] * smooth[e]),
// scale = fl32(max|xs| / qmax), codes of fl32(xs / scale).  Each copy gets
// its own row and scale.  One workgroup per token; the token's row stays in
// VGPRs (as bf16) while the copies are quantised one after another, each
// copy's smoothing row read from L2 (E x H fp32 is shared by all tokens).
// ---------------------------------------------------------------------------
template <int QT, int G, bool NTS>
__global__ __launch_bounds__(kRowThreads) void dispatch_smooth_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids, const int32_t* __restrict__ pos,
    const float4* __restrict__ smooth, u32x4* __restrict__ q, float* __restrict__ scales, int T, int K,
    int E, int NG, int64_t cap_rows) {
  __shared__ uint32_t s_max[2][kRowThreads / kWave];  // alternate copies use alternate halves
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int my_pos = row_of(pos, t, K, lane, cap_rows);
  const int my_e = lane < K ? ids[(int64_t)t * K + lane] : -1;
  const uint64_t live = ballot(my_pos >= 0 && (unsigned)my_e < (unsigned)E);
  if (ballot(my_pos >= 0 && (unsigned)my_e >= (unsigned)E) && lane == 0) raise_device_error(kErrBadExpert);
  if (live == 0) return;
  const u32x4* src = x + (int64_t)t * NG * 2;
  // The token's values as fp32, unpacked once for all of its copies.
  float xf[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = g * kRowThreads + tid;
    u32x4 a = u32x4{0, 0, 0, 0}, b = u32x4{0, 0, 0, 0};
    if (idx < NG) {
      a = src[2 * idx];
      b = src[2 * idx + 1];
    }
    unpack16(a, b, xf[g]);
  }
  uint64_t mk = live;
  int half = 0;
  while (mk) {
    const int k = __builtin_ctzll(mk);
    mk &= mk - 1;
    const int p = __builtin_amdgcn_readlane(my_pos, k);
    const int e = __builtin_amdgcn_readlane(my_e, k);
    const float4* srow = smooth + (int64_t)e * NG * 4;
    float xs[G][16];
    float amax = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = g * kRowThreads + tid;
      if (idx < NG) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const float4 sv = srow[4 * idx + qd];
          xs[g][4 * qd + 0] = xf[g][4 * qd + 0] * sv.x;
          xs[g][4 * qd + 1] = xf[g][4 * qd + 1] * sv.y;
          xs[g][4 * qd + 2] = xf[g][4 * qd + 2] * sv.z;
          xs[g][4 * qd + 3] = xf[g][4 * qd + 3] * sv.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(xs[g][j]));
      }
    }
    // Copy c's wave maxima go to half c % 2: the barrier of copy c + 1
    // follows every wave's reads of copy c, so half c % 2 is free again
    // when copy c + 2 writes it.
    const uint32_t mb = wave_max_u32(__float_as_uint(amax));
    if (lane == 0) s_max[half][wave] = mb;
    __syncthreads();
    uint32_t m = s_max[half][0];
#pragma unroll
    for (int w = 1; w < kRowThreads / kWave; ++w) m = max(m, s_max[half][w]);
    half ^= 1;
    const float scale = __uint_as_float(m) / quant_max<QT>();
    const RowDiv rd = row_div(scale);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = g * kRowThreads + tid;
      if (idx < NG) st<NTS>(q + (int64_t)p * NG + idx, quantize16r<QT>(xs[g], rd));
    }
    if (tid == 0) scales[p] = scale;
  }
}

// ---------------------------------------------------------------------------
// Combine of quantised expert rows (commQuantMode of the CANN combine): row
// values are decode(code) * row_scale in fp32, then summed with the gate
// weights as ep_combine does.  Work item: one wavefront per (token, chunk of
// 1024 columns); a lane reads 16 codes (16 bytes) of each of the K rows.
// ---------------------------------------------------------------------------
// Four codes of one dword (byte i is code i) as fp32 values.  fp8:
// v_cvt_pk_f32_fp8 decodes OCP E4M3FN codes exactly (all 256 codes compared
// with the format's definition: sign, 4-bit exponent of bias 7, 3-bit
// mantissa, subnormals below exponent 1; the two NaN codes give a NaN).
template <int QT>
__device__ __forceinline__ void decode4(uint32_t c, float* v) {
  if constexpr (QT == kQFp8) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
    const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
    v[0] = lo.x;
    v[1] = lo.y;
    v[2] = hi.x;
    v[3] = hi.y;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (float)(int32_t)(int8_t)((c >> (8 * j)) & 0xffu);
  }
}

template <int QT, int KMAX, int WPB, bool NTL, bool NTS>
__global__ __launch_bounds__(WPB * kWave) void combine_quant_kernel(
    const u32x4* __restrict__ codes, const float* __restrict__ row_scales,
    const int32_t* __restrict__ pos, const float* __restrict__ w, u32x4* __restrict__ out, int T,
    int K, int NG, int chunks, int64_t cap_rows) {
  const int64_t g = (int64_t)blockIdx.x * WPB + uniform((int)(threadIdx.x / kWave));
  const int64_t t64 = g / chunks;
  if (t64 >= T) return;
  const int t = (int)t64;
  const int idx = (int)(g - t64 * chunks) * kWave + lane_id();
  const int lane = lane_id();
  const int my_pos = row_of(pos, t, K, lane, cap_rows);
  const float my_w = lane < K ? w[(int64_t)t * K + lane] : 0.0f;
  const float my_s = my_pos >= 0 ? row_scales[my_pos] : 0.0f;
  int pk[KMAX];
  float wk[KMAX], sk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    pk[k] = __builtin_amdgcn_readlane(my_pos, k);
    wk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k));
    sk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
  }
  if (idx >= NG) return;
  u32x4 r[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (pk[k] >= 0) r[k] = ld<NTL>(codes + (int64_t)pk[k] * NG + idx);
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (pk[k] >= 0) {
      const uint32_t c4[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[4];
        decode4<QT>(c4[i], v);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * i + j] = __builtin_fmaf(wk[k], v[j] * sk[k], acc[4 * i + j]);
      }
    }
  }
  u32x4 o0, o1;
  o0.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o0.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o0.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o0.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  o1.x = f32_to_bf16_rne(acc[8]) | (f32_to_bf16_rne(acc[9]) << 16);
  o1.y = f32_to_bf16_rne(acc[10]) | (f32_to_bf16_rne(acc[11]) << 16);
  o1.z = f32_to_bf16_rne(acc[12]) | (f32_to_bf16_rne(acc[13]) << 16);
  o1.w = f32_to_bf16_rne(acc[14]) | (f32_to_bf16_rne(acc[15]) << 16);
  u32x4* dst = out + (int64_t)t * NG * 2;
  st<NTS>(dst + 2 * idx, o0);
  st<NTS>(dst + 2 * idx + 1, o1);
}

// ---------------------------------------------------------------------------
// Combine fused with the layer tail: residual add and RMSNorm (the
// MoE-finalize + residual + RMSNorm pattern of flashinfer PR #4358, without
// the all-reduce; CombineAddRmsNorm on the CANN dispatch page):
//   c = bf16(sum_k w[t][k] y[pos[t][k]]),  h = bf16(residual[t] + c),
//   norm = bf16(h * gamma / sqrt(mean(h^2) + eps)).
// One NT-thread workgroup per token; thread i owns the 16-byte vectors i,
// i + NT, ... (NV of them, H <= NV * NT * 8), whose h values stay in VGPRs
// between the sum-of-squares pass and the scaling pass.  The combined rows
// never go to HBM.  With y == nullptr the kernel is the tail alone: c = x[t].
// ---------------------------------------------------------------------------
template <int KMAX, int NV, int NT, bool NTL, bool NTS>
__global__ __launch_bounds__(NT) void combine_add_rmsnorm_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    const u32x4* __restrict__ x, const u32x4* __restrict__ residual, const u32x4* __restrict__ gamma,
    float eps, u32x4* __restrict__ residual_out, u32x4* __restrict__ norm_out, int T, int K, int V,
    int64_t cap_rows) {
  __shared__ float s_sum[NT / kWave];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  int pk[KMAX];
  float wk[KMAX];
  if (y != nullptr) {
    const int my_pos = row_of(pos, t, K, lane, cap_rows);
    const float my_w = lane < K ? w[(int64_t)t * K + lane] : 0.0f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      pk[k] = __builtin_amdgcn_readlane(my_pos, k);
      wk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k));
    }
  }
  float hv[NV][8];
  float sumsq = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * NT;
    if (v < V) {
      float c[8];
      if (y != nullptr) {
        u32x4 r[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (pk[k] >= 0) r[k] = ld<NTL>(y + (int64_t)pk[k] * V + v);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          if (pk[k] >= 0) {
            const uint32_t v4[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              c[2 * j] = __builtin_fmaf(wk[k], bf16lo(v4[j]), c[2 * j]);
              c[2 * j + 1] = __builtin_fmaf(wk[k], bf16hi(v4[j]), c[2 * j + 1]);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __uint_as_float(f32_to_bf16_rne(c[j]) << 16);
      } else {
        const u32x4 xv = ld<NTL>(x + (int64_t)t * V + v);
        const uint32_t v4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[2 * j] = bf16lo(v4[j]);
          c[2 * j + 1] = bf16hi(v4[j]);
        }
      }
      const u32x4 rv = ld<NTL>(residual + (int64_t)t * V + v);
      const uint32_t r4[4] = {rv.x, rv.y, rv.z, rv.w};
      uint32_t hb[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hb[2 * j] = f32_to_bf16_rne(bf16lo(r4[j]) + c[2 * j]);
        hb[2 * j + 1] = f32_to_bf16_rne(bf16hi(r4[j]) + c[2 * j + 1]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hv[i][j] = __uint_as_float(hb[j] << 16);
        sumsq = __builtin_fmaf(hv[i][j], hv[i][j], sumsq);
      }
      u32x4 o;
      o.x = hb[0] | (hb[1] << 16);
      o.y = hb[2] | (hb[3] << 16);
      o.z = hb[4] | (hb[5] << 16);
      o.w = hb[6] | (hb[7] << 16);
      st<NTS>(residual_out + (int64_t)t * V + v, o);
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) sumsq += __shfl_xor(sumsq, off, kWave);
  if (lane == 0) s_sum[wave] = sumsq;
  __syncthreads();
  float total = 0.0f;
#pragma unroll
  for (int q = 0; q < NT / kWave; ++q) total += s_sum[q];
  const float inv = 1.0f / sqrtf(total / (float)(V * 8) + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * NT;
    if (v < V) {
      const u32x4 gv = gamma[v];
      const uint32_t g4[4] = {gv.x, gv.y, gv.z, gv.w};
      uint32_t nb[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        nb[2 * j] = f32_to_bf16_rne(hv[i][2 * j] * inv * bf16lo(g4[j]));
        nb[2 * j + 1] = f32_to_bf16_rne(hv[i][2 * j + 1] * inv * bf16hi(g4[j]));
      }
      u32x4 o;
      o.x = nb[0] | (nb[1] << 16);
      o.y = nb[2] | (nb[3] << 16);
      o.z = nb[4] | (nb[5] << 16);
      o.w = nb[6] | (nb[7] << 16);
      st<NTS>(norm_out + (int64_t)t * V + v, o);
    }
  }
}

// ---------------------------------------------------------------------------
// 1-D uneven all_to_all_single (test_make_a2a_exchange_plan / allToAllGet on
// the PyTorch compare view; aws-neuron/torch-neuronx PR #1035).
// ---------------------------------------------------------------------------
constexpr int kSplitsPlanThreads = 64;

__global__ __launch_bounds__(kSplitsPlanThreads) void plan_splits_kernel(
    int W, const int64_t* __restrict__ in_splits, int64_t* __restrict__ src_offsets,
    int64_t* __restrict__ out_splits, int64_t* __restrict__ dst_offsets,
    int64_t* __restrict__ rank_offsets) {
  __shared__ int64_t recv[kSplitsPlanThreads];
  const int r = threadIdx.x;  // receiver
  if (r < W) {
    int64_t run = 0;
    for (int p = 0; p < W; ++p) {
      const int64_t n = in_splits[(int64_t)p * W + r];
      out_splits[(int64_t)r * W + p] = n;
      dst_offsets[(int64_t)r * W + p] = run;
      run += n;
      int64_t so = 0;
      for (int r2 = 0; r2 < r; ++r2) so += in_splits[(int64_t)p * W + r2];
      src_offsets[(int64_t)r * W + p] = so;
    }
    recv[r] = run;
  }
  __syncthreads();
  if (r == 0) {
    int64_t run = 0;
    for (int i = 0; i < W; ++i) {
      rank_offsets[i] = run;
      run += recv[i];
    }
    rank_offsets[W] = run;
  }
}

// Grid: x = chunk q = r * W + p (receiver r, sender p), y = blocks per chunk.
// Each wave copies whole rows of its chunk, 16-byte vectors, U per lane.
template <int U, bool NTL, bool NTS>
__global__ __launch_bounds__(kRowThreads) void copy_splits_kernel(
    const u32x4* __restrict__ in, u32x4* __restrict__ out, const int64_t* __restrict__ src_offsets,
    const int64_t* __restrict__ out_splits, const int64_t* __restrict__ dst_offsets,
    const int64_t* __restrict__ rank_offsets, int W, int64_t R, int64_t Vr) {
  const int q = blockIdx.x;
  const int r = q / W, p = q - r * W;
  const int64_t n = out_splits[q];
  const int64_t src = src_offsets[q];
  const int64_t dst = rank_offsets[r] + dst_offsets[q];
  if (n == 0) return;
  if (n < 0 || src < 0 || src + n > R || dst < 0 || dst + n > (int64_t)W * R) {
    if (blockIdx.y == 0 && threadIdx.x == 0) raise_device_error(kErrSplits);
    return;
  }
  const int lane = lane_id();
  const int64_t step = (int64_t)gridDim.y * kTokensPerBlock;
  for (int64_t i = (int64_t)blockIdx.y * kTokensPerBlock + threadIdx.x / kWave; i < n; i += step) {
    const u32x4* s = in + ((int64_t)p * R + src + i) * Vr;
    u32x4* d = out + (dst + i) * Vr;
    for (int64_t v0 = 0; v0 < Vr; v0 += kWave * U) {
      u32x4 t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t idx = v0 + u * kWave + lane;
        if (idx < Vr) t[u] = ld<NTL>(s + idx);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t idx = v0 + u * kWave + lane;
        if (idx < Vr) st<NTS>(d + idx, t[u]);
      }
    }
  }
}

// The plan and the data move of the 1-D all-to-all in one launch, balanced
// by rows.  The send matrix in_splits[p][r] (sender p, receiver r; W*W
// values) is staged in LDS by every workgroup, which derives from it
//   rank_offsets[r] = sum_{r' < r} sum_p in_splits[p][r']   (receiver bases)
// and checks that every entry is >= 0 and every sender's row sums to at most
// R.  Such a matrix places every chunk inside the buffers, and the output is
// the W*R-row space [0, rank_offsets[W]) covered by the chunks back to back,
// so the work is split by output rows into ranges of RPB = 4 RPW rows:
// workgroup b copies ranges b, b + gridDim.x, ..., each wave of it a
// contiguous run of RPW rows of the range.  A wave finds
// the chunk of its first row (and again whenever it crosses into the next):
//   r = number of receivers r' >= 1 with rank_offsets[r'] <= o,
//   p = number of senders whose inclusive prefix of column r is <= o - rank_offsets[r],
//   src = sum_{r' < r} in_splits[p][r'] + (o - start of (r, p)'s chunk),
// from lane-parallel scans over the W <= 64 lanes of the wave.  Every chunk
// thus gets waves in proportion to its rows (a fixed number of workgroups
// per chunk leaves the largest chunks' waves copying long after the rest).
// Any other matrix (a negative entry, a row summing past R) takes the
// chunk-by-chunk form: each chunk's offsets are derived as above from the
// prefix sums, a chunk reaching outside the buffers is skipped and raises
// kErrSplits, and the workgroups take chunks in turn.  Workgroup b < W
// also writes receiver b's row of the plan (each output may be null).
constexpr int kA2ARowsPerWaveBytes = 4096;  // bytes a wave copies per run
constexpr int64_t kA2ABlocks = 1024;          // workgroups of one launch

template <int U, bool NTL, bool NTS>
__device__ __forceinline__ void copy_row(const u32x4* __restrict__ s, u32x4* __restrict__ d, int64_t Vr, int lane) {
  for (int64_t v0 = 0; v0 < Vr; v0 += kWave * U) {
    u32x4 t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = v0 + u * kWave + lane;
      if (idx < Vr) t[u] = ld<NTL>(s + idx);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = v0 + u * kWave + lane;
      if (idx < Vr) st<NTS>(d + idx, t[u]);
    }
  }
}

template <int U, bool NTL, bool NTS>
__global__ __launch_bounds__(kRowThreads) void all_to_all_splits_kernel(
    const u32x4* __restrict__ in, u32x4* __restrict__ out, const int64_t* __restrict__ in_splits,
    int64_t* __restrict__ src_offsets, int64_t* __restrict__ out_splits, int64_t* __restrict__ dst_offsets,
    int64_t* __restrict__ rank_offsets, int W, int64_t R, int64_t Vr, int64_t rows_per_wave,
    int64_t n_ranges) {
  extern __shared__ int64_t a2a_lds[];
  int64_t* cnt = a2a_lds;              // [W][W] send matrix, sender-major
  int64_t* base = a2a_lds + W * W;     // [W + 1] receiver bases (rank_offsets)
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  if (tid == 0) s_bad = 0;
  for (int e = tid; e < W * W; e += kRowThreads) cnt[e] = in_splits[e];
  __syncthreads();
  if (tid < W) {  // receiver tid's column sum; sender tid's row check
    int64_t col = 0, row = 0;
    bool neg = false;
    for (int q = 0; q < W; ++q) {
      const int64_t c = cnt[(int64_t)q * W + tid], rv = cnt[(int64_t)tid * W + q];
      col += c;
      row += rv;
      neg |= c < 0;
    }
    base[tid + 1] = col;
    if (neg || row > R) s_bad = 1;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    base[0] = 0;
    for (int r = 0; r < W; ++r) {
      run += base[r + 1];
      base[r + 1] = run;
    }
  }
  __syncthreads();

  // Receiver b's row of the plan.
  for (int r = blockIdx.x; r < W; r += gridDim.x) {
    for (int p = tid; p < W; p += kRowThreads) {
      int64_t so = 0, dsub = 0;
      for (int q = 0; q < r; ++q) so += cnt[(int64_t)p * W + q];
      for (int q = 0; q < p; ++q) dsub += cnt[(int64_t)q * W + r];
      const int64_t j = (int64_t)r * W + p;
      if (out_splits) out_splits[j] = cnt[(int64_t)p * W + r];
      if (src_offsets) src_offsets[j] = so;
      if (dst_offsets) dst_offsets[j] = dsub;
    }
    if (rank_offsets && tid == 0) rank_offsets[r] = base[r];
  }
  if (rank_offsets && blockIdx.x == 0 && tid == 0) rank_offsets[W] = base[W];
  if (R == 0) return;

  if (!s_bad) {
    const int64_t total = base[W];
    for (int64_t g = blockIdx.x; g < n_ranges; g += gridDim.x) {
      int64_t o = (g * (kRowThreads / kWave) + wave) * rows_per_wave;
      const int64_t o_end = min(o + rows_per_wave, total);
      int64_t chunk_end = -1, shift = 0;  // input row of output row o: o + shift
      for (; o < o_end; ++o) {
        if (o >= chunk_end) {
          // receiver of row o
          const bool past = lane >= 1 && lane <= W && base[lane] <= o;
          const int r = __popcll(ballot(past));
          const int64_t orr = o - base[r];
          // sender: inclusive prefix of column r over the lanes
          const int64_t c = lane < W ? cnt[(int64_t)lane * W + r] : 0;
          int64_t incl = c;
#pragma unroll
          for (int off = 1; off < kWave; off <<= 1) {
            const int64_t v = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += v;
          }
          const int p = __popcll(ballot(lane < W && incl <= orr));
          const int64_t incl_p = __shfl(incl, p, kWave);
          const int64_t n_p = __shfl(c, p, kWave);
          // rows sender p sends to receivers before r
          int64_t so = lane < r ? cnt[(int64_t)p * W + lane] : 0;
#pragma unroll
          for (int off = kWave / 2; off > 0; off >>= 1) so += __shfl_xor(so, off, kWave);
          const int64_t chunk_start = base[r] + incl_p - n_p;
          chunk_end = base[r] + incl_p;
          shift = (int64_t)p * R + so - chunk_start;
        }
        copy_row<U, NTL, NTS>(in + (o + shift) * Vr, out + o * Vr, Vr, lane);
      }
    }
    return;
  }

  // Chunk by chunk (a matrix that does not place every chunk inside the
  // buffers): the checks and skips of ep_dispatch_splits.
  for (int q = blockIdx.x; q < W * W; q += gridDim.x) {
    const int r = q / W, p = q - r * W;
    const int64_t n = cnt[(int64_t)p * W + r];
    if (n == 0) continue;
    int64_t so = 0, dsub = 0;
    for (int j = 0; j < r; ++j) so += cnt[(int64_t)p * W + j];
    for (int j = 0; j < p; ++j) dsub += cnt[(int64_t)j * W + r];
    const int64_t dst = base[r] + dsub;
    if (n < 0 || so < 0 || so + n > R || dst < 0 || dst + n > (int64_t)W * R) {
      if (tid == 0) raise_device_error(kErrSplits);
      continue;
    }
    for (int64_t i = wave; i < n; i += kRowThreads / kWave)
      copy_row<U, NTL, NTS>(in + ((int64_t)p * R + so + i) * Vr, out + (dst + i) * Vr, Vr, lane);
  }
}

}  // namespace ep
