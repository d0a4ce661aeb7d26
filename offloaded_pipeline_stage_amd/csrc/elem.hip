// Row-wise and elementwise kernels of the stage: RMSNorm forward/backward,
// RoPE, SwiGLU (for the unfused fp32 path), the vocabulary-sharded
// cross-entropy, token embedding. All HBM-bound: one wavefront per row with
// 16-byte vector accesses, reductions by fixed-order butterflies so every
// result is deterministic (recomputation must reproduce the forward exactly).
#include <type_traits>
#include <algorithm>

#include "ops.h"
#include "trace.h"

namespace rp {
namespace {

// 16-byte vector of VEC elements
template <class T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; typedef float4 type; };
template <> struct Vec<bf16> { static constexpr int N = 8; typedef uint4 type; };

template <class T>
__device__ __forceinline__ void load_vec(const T* p, float* out);
template <>
__device__ __forceinline__ void load_vec<float>(const float* p, float* out) {
  float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <>
__device__ __forceinline__ void load_vec<bf16>(const bf16* p, float* out) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <class T>
__device__ __forceinline__ void store_vec(T* p, const float* in);
template <>
__device__ __forceinline__ void store_vec<float>(float* p, const float* in) {
  *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
}
template <>
__device__ __forceinline__ void store_vec<bf16>(bf16* p, const float* in) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = uint32_t(to_bf16(in[2 * i]).u) | (uint32_t(to_bf16(in[2 * i + 1]).u) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// V consecutive elements of type T as floats (16-byte loads where they fit)
template <class T, int V>
__device__ __forceinline__ void load_n(const T* p, float* out) {
  if constexpr (Vec<T>::N <= V) {
#pragma unroll
    for (int q = 0; q < V; q += Vec<T>::N) load_vec<T>(p + q, out + q);
  } else {
#pragma unroll
    for (int q = 0; q < V; ++q) out[q] = to_f(p[q]);
  }
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// plain 16-byte-per-lane copy: the reference that HBM byte counters are
// scaled by, with the same load and store width as the library's kernels
__global__ void copy16_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n16) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) dst[i] = src[i];
}

// fp32 -> bf16, rounded to nearest even: 8 values (32 bytes in, 16 out) per
// lane and step
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, to_bf16(lo)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, to_bf16(hi)) << 16);
}
__global__ __launch_bounds__(256) void convert_f32_bf16_kernel(uint4* __restrict__ dst, const float4* __restrict__ src,
                                                            size_t n8) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n8; i += stride) {
    const float4 a = src[2 * i], b = src[2 * i + 1];
    dst[i] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
  }
}

// ---------------------------------------------------------------------------
// RMSNorm
// ---------------------------------------------------------------------------

// one wave per row; 4 rows per 256-thread block
template <class T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ gamma,
                                                          T* __restrict__ y, float* __restrict__ rstd,
                                                          int rows, int H, float eps) {
  constexpr int V = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + (int64_t)row * H;
  float ss = 0.f;
  for (int c = lane * V; c < H; c += 64 * V) {
    float v[V];
    load_vec<T>(xr + c, v);
#pragma unroll
    for (int i = 0; i < V; ++i) ss = fmaf(v[i], v[i], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (lane == 0) rstd[row] = r;
  T* yr = y + (int64_t)row * H;
  for (int c = lane * V; c < H; c += 64 * V) {
    float v[V], g[V];
    load_vec<T>(xr + c, v);
    load_vec<T>(gamma + c, g);
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = v[i] * r * g[i];
    store_vec<T>(yr + c, v);
  }
}

// The same for bf16 rows of NV * 512 elements, the row held in registers:
// each row is read from memory once (the two-pass kernel above reads it twice,
// and its second read misses L2), every lane's loads issued together. The
// lane owns the same elements and sums their squares in the same order, so
// the results are bit-identical.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_fwd_rows_kernel(const bf16* __restrict__ x,
                                                               const bf16* __restrict__ gamma,
                                                               bf16* __restrict__ y, float* __restrict__ rstd,
                                                               int rows, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bf16* xr = x + (int64_t)row * H;
  float v[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) load_vec<bf16>(xr + (64 * j + lane) * 8, v[j]);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[j][i], v[j][i], ss);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (lane == 0) rstd[row] = r;
  bf16* yr = y + (int64_t)row * H;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float g[8];
    load_vec<bf16>(gamma + (64 * j + lane) * 8, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[j][i] = v[j][i] * r * g[i];
    store_vec<bf16>(yr + (64 * j + lane) * 8, v[j]);
  }
}

// dx = r*(g*gamma) - x * r^3 * mean(g*gamma*x) + resid
// Each block owns RB consecutive rows (one wave per row at a time) and writes
// its dgamma partial row; a second kernel sums the partials in block order.
constexpr int RMS_BWD_ROWS = 16;

template <class T, class TR>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(
    const float* __restrict__ g, const T* __restrict__ x, const T* __restrict__ gamma,
    const float* __restrict__ rstd, const TR* __restrict__ resid, float* __restrict__ out_f32,
    T* __restrict__ out_dt, float* __restrict__ part, int rows, int H) {
  constexpr int V = Vec<T>::N;
  extern __shared__ float sm[];  // [4][H] wave partials of dgamma
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* my = sm + wave * H;
  for (int c = lane; c < H; c += 64) my[c] = 0.f;
  const int r0 = blockIdx.x * RMS_BWD_ROWS;
  for (int rr = wave; rr < RMS_BWD_ROWS; rr += 4) {
    const int row = r0 + rr;
    if (row >= rows) break;
    const float r = rstd[row];
    const T* xr = x + (int64_t)row * H;
    const float* gr = g + (int64_t)row * H;
    float dot = 0.f;
    for (int c = lane * V; c < H; c += 64 * V) {
      float xv[V], gm[V];
      load_vec<T>(xr + c, xv);
      load_vec<T>(gamma + c, gm);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float gv = gr[c + i];
        dot = fmaf(gv * gm[i], xv[i], dot);
        my[c + i] += gv * xv[i] * r;
      }
    }
    dot = wave_sum(dot);
    const float coef = r * r * r * dot / (float)H;
    for (int c = lane * V; c < H; c += 64 * V) {
      float xv[V], gm[V], o[V];
      load_vec<T>(xr + c, xv);
      load_vec<T>(gamma + c, gm);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float v = r * gr[c + i] * gm[i] - xv[i] * coef;
        if (resid) v += to_f(resid[(int64_t)row * H + c + i]);
        o[i] = v;
      }
      if (out_f32) {
#pragma unroll
        for (int i = 0; i < V; ++i) out_f32[(int64_t)row * H + c + i] = o[i];
      }
      if (out_dt) store_vec<T>(out_dt + (int64_t)row * H + c, o);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H; c += 256)
    part[(int64_t)blockIdx.x * H + c] = sm[c] + sm[H + c] + sm[2 * H + c] + sm[3 * H + c];
}

// RMSNorm backward with the row in registers (H = 64 V NC): lane l owns the
// columns (64 j + l) V .. + V - 1 for j < NC; a row is loaded once, all its
// loads issued together. Each wave sums its share of dgamma over its rows
// (wave, wave + 4 gridDim, ...) in its own LDS row (16-byte read-modify-
// writes of the lane's own columns); the block's four rows are then added
// into one partial row. Same per-row arithmetic as rmsnorm_bwd_kernel.
template <class T, class TR, int NC>
__global__ __launch_bounds__(256) void rmsnorm_bwd_rows_kernel(
    const float* __restrict__ g, const T* __restrict__ x, const T* __restrict__ gamma,
    const float* __restrict__ rstd, const TR* __restrict__ resid, float* __restrict__ out_f32,
    T* __restrict__ out_dt, float* __restrict__ part, int rows) {
  constexpr int V = Vec<T>::N, H = 64 * V * NC;
  typedef typename Vec<T>::type VT;
  extern __shared__ float sm[];  // [4][H]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* my = sm + wave * H;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int q = 0; q < V; q += 4)
      *reinterpret_cast<float4*>(my + (64 * j + lane) * V + q) = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int row = blockIdx.x * 4 + wave; row < rows; row += gridDim.x * 4) {
    const float r = rstd[row];
    const int64_t ro = (int64_t)row * H;
    VT xr[NC];  // x as loaded (16 bytes per chunk)
    float gv[NC][V];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = (64 * j + lane) * V;
      xr[j] = *reinterpret_cast<const VT*>(x + ro + c);
#pragma unroll
      for (int q = 0; q < V; q += 4) {
        const float4 v = *reinterpret_cast<const float4*>(g + ro + c + q);
        gv[j][q] = v.x; gv[j][q + 1] = v.y; gv[j][q + 2] = v.z; gv[j][q + 3] = v.w;
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float xv[V], gm[V];
      load_vec<T>(reinterpret_cast<const T*>(&xr[j]), xv);
      load_vec<T>(gamma + (64 * j + lane) * V, gm);
#pragma unroll
      for (int i = 0; i < V; ++i) dot = fmaf(gv[j][i] * gm[i], xv[i], dot);
    }
    dot = wave_sum(dot);
    const float coef = r * r * r * dot / (float)H;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = (64 * j + lane) * V;
      float xv[V], gm[V], o[V];
      load_vec<T>(reinterpret_cast<const T*>(&xr[j]), xv);
      load_vec<T>(gamma + c, gm);
      float rv[V];
      if (resid) load_n<TR, V>(resid + ro + c, rv);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float v = r * gv[j][i] * gm[i] - xv[i] * coef;
        if (resid) v += rv[i];
        o[i] = v;
      }
#pragma unroll
      for (int q = 0; q < V; q += 4) {
        float4* a = reinterpret_cast<float4*>(my + c + q);
        float4 t = *a;
        t.x += gv[j][q] * xv[q] * r;
        t.y += gv[j][q + 1] * xv[q + 1] * r;
        t.z += gv[j][q + 2] * xv[q + 2] * r;
        t.w += gv[j][q + 3] * xv[q + 3] * r;
        *a = t;
      }
      if (out_f32) {
#pragma unroll
        for (int q = 0; q < V; q += 4)
          *reinterpret_cast<float4*>(out_f32 + ro + c + q) = make_float4(o[q], o[q + 1], o[q + 2], o[q + 3]);
      }
      if (out_dt) store_vec<T>(out_dt + ro + c, o);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H; c += 256)
    part[(int64_t)blockIdx.x * H + c] = sm[c] + sm[H + c] + sm[2 * H + c] + sm[3 * H + c];
}

// column sums of a [nrow][H] matrix: 32 columns x 8 row slices per block,
// each slice summed in row order, the slices in a fixed order; `accumulate`
// adds the sums to out instead of overwriting it
__global__ __launch_bounds__(256) void sum_rows_kernel(const float* __restrict__ part, int nrow, int H,
                                                       float* __restrict__ out, int accumulate) {
  __shared__ float red[8][33];
  const int cx = threadIdx.x & 31, sy = threadIdx.x >> 5;
  const int c = blockIdx.x * 32 + cx;
  float s = 0.f;
  if (c < H)
    for (int r = sy; r < nrow; r += 8) s += part[(int64_t)r * H + c];
  red[sy][cx] = s;
  __syncthreads();
  if (sy == 0 && c < H) {
    float t = red[0][cx];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += red[k][cx];
    out[c] = accumulate ? out[c] + t : t;
  }
}

// ---------------------------------------------------------------------------
// RoPE (rotate-half pairs (i, i + d/2))
// ---------------------------------------------------------------------------

__global__ void rope_table_kernel(float2* tab, int seq, int d, double base) {
  const int half = d / 2;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)seq * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(base, -2.0 * (double)i / (double)d);
  const double th = (double)p * inv;
  tab[idx] = make_float2((float)cos(th), (float)sin(th));
}

// one thread per (row, head, pair)
template <class T>
__global__ void rope_apply_kernel(T* buf, int64_t ld, int rows, int seq, int n_heads, int d,
                                  const float2* __restrict__ tab, int inverse) {
  const int half = d / 2;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)n_heads * half;
  if (idx >= (int64_t)rows * per_row) return;
  const int row = (int)(idx / per_row);
  const int rem = (int)(idx % per_row);
  const int h = rem / half, i = rem % half;
  const int p = row % seq;
  const float2 cs = tab[(int64_t)p * half + i];
  const float s = inverse ? -cs.y : cs.y;
  T* base = buf + (int64_t)row * ld + (int64_t)h * d;
  const float a = to_f(base[i]), b = to_f(base[i + half]);
  base[i] = from_f<T>(a * cs.x - b * s);
  base[i + half] = from_f<T>(b * cs.x + a * s);
}

// The same rotation for bf16 buffers, four pairs per thread: 8-byte loads
// and stores of each half, the four (cos, sin) pairs in two 16-byte loads.
// Needs d % 8 == 0, ld % 4 == 0 and an 8-byte aligned buffer.
__global__ void rope_apply4_kernel(bf16* buf, int64_t ld, int rows, int seq, int n_heads, int d,
                                   const float2* __restrict__ tab, int inverse) {
  const int half = d / 2, q = half / 4;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)n_heads * q;
  if (idx >= (int64_t)rows * per_row) return;
  const int row = (int)(idx / per_row);
  const int rem = (int)(idx % per_row);
  const int h = rem / q, i0 = 4 * (rem % q);
  const int p = row % seq;
  const float4 t01 = *reinterpret_cast<const float4*>(tab + (int64_t)p * half + i0);
  const float4 t23 = *reinterpret_cast<const float4*>(tab + (int64_t)p * half + i0 + 2);
  const float c[4] = {t01.x, t01.z, t23.x, t23.z};
  float sn[4] = {t01.y, t01.w, t23.y, t23.w};
  if (inverse)
#pragma unroll
    for (int e = 0; e < 4; ++e) sn[e] = -sn[e];
  bf16* base = buf + (int64_t)row * ld + (int64_t)h * d + i0;
  const uint2 ua = *reinterpret_cast<const uint2*>(base);
  const uint2 ub = *reinterpret_cast<const uint2*>(base + half);
  const uint32_t wa[2] = {ua.x, ua.y}, wb[2] = {ub.x, ub.y};
  uint32_t oa[2], ob[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float a2[2], b2[2], ra[2], rb[2];
    a2[0] = __uint_as_float(wa[k] << 16); a2[1] = __uint_as_float(wa[k] & 0xffff0000u);
    b2[0] = __uint_as_float(wb[k] << 16); b2[1] = __uint_as_float(wb[k] & 0xffff0000u);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      ra[e] = a2[e] * c[2 * k + e] - b2[e] * sn[2 * k + e];
      rb[e] = b2[e] * c[2 * k + e] + a2[e] * sn[2 * k + e];
    }
    oa[k] = (uint32_t)to_bf16(ra[0]).u | ((uint32_t)to_bf16(ra[1]).u << 16);
    ob[k] = (uint32_t)to_bf16(rb[0]).u | ((uint32_t)to_bf16(rb[1]).u << 16);
  }
  *reinterpret_cast<uint2*>(base) = make_uint2(oa[0], oa[1]);
  *reinterpret_cast<uint2*>(base + half) = make_uint2(ob[0], ob[1]);
}

// ---------------------------------------------------------------------------
// SwiGLU (unfused path)
// ---------------------------------------------------------------------------
template <class T>
__global__ void swiglu_fwd_kernel(const T* gu, T* m, int rows, int F) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * F) return;
  const int64_t t = idx / F, f = idx % F;
  const float g = to_f(gu[t * 2 * F + f]), u = to_f(gu[t * 2 * F + F + f]);
  m[idx] = from_f<T>(g / (1.f + expf(-g)) * u);
}

template <class T>
__global__ void swiglu_bwd_kernel(const float* dm, const T* gu, T* dgu, int rows, int F) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * F) return;
  const int64_t t = idx / F, f = idx % F;
  const float g = to_f(gu[t * 2 * F + f]), u = to_f(gu[t * 2 * F + F + f]);
  const float sg = 1.f / (1.f + expf(-g));
  const float v = dm[idx];
  dgu[t * 2 * F + f] = from_f<T>(v * u * sg * (1.f + g * (1.f - sg)));
  dgu[t * 2 * F + F + f] = from_f<T>(v * g * sg);
}

// ---------------------------------------------------------------------------
// cross-entropy
// ---------------------------------------------------------------------------

// merge (m, l) <- (m, l) + values v: l is the sum of exp(x - m) over the
// values seen so far (m = -inf, l = 0 before the first)
__device__ __forceinline__ void lse_merge4(float& m, float& l, float4 v) {
  const float mn = fmaxf(fmaxf(m, fmaxf(v.x, v.y)), fmaxf(v.z, v.w));
  l = l * __expf(m - mn) + __expf(v.x - mn) + __expf(v.y - mn) + __expf(v.z - mn) + __expf(v.w - mn);
  m = mn;
}
__device__ __forceinline__ void lse_merge1(float& m, float& l, float v) {
  const float mn = fmaxf(m, v);
  l = l * __expf(m - mn) + __expf(v - mn);
  m = mn;
}

// one wave per row: online (max, sum-exp) over the shard's logits. VEC: the
// row is read as 16-byte vectors, four in flight per lane (row starts 16-byte
// aligned), the ragged end one value per lane.
template <bool VEC>
__global__ __launch_bounds__(256) void ce_stats_kernel(const float* __restrict__ z, int64_t ld, int rows,
                                                       int Vs, int vlo, const int32_t* __restrict__ labels,
                                                       int vocab, float2* part, float* zlab) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* zr = z + (int64_t)row * ld;
  float m = -INFINITY, l = 0.f;
  int c0 = 0;
  if constexpr (VEC) {
    const float4* z4 = reinterpret_cast<const float4*>(zr);
    const int n4 = Vs >> 2;
    int c = lane;
    for (; c + 192 < n4; c += 256) {
      const float4 a = z4[c], b = z4[c + 64], d = z4[c + 128], e = z4[c + 192];
      lse_merge4(m, l, a);
      lse_merge4(m, l, b);
      lse_merge4(m, l, d);
      lse_merge4(m, l, e);
    }
    for (; c < n4; c += 64) lse_merge4(m, l, z4[c]);
    c0 = n4 << 2;
  }
  for (int c = c0 + lane; c < Vs; c += 64) lse_merge1(m, l, zr[c]);
  // merge lanes in butterfly order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o, 64), lo = __shfl_xor(l, o, 64);
    const float mn = fmaxf(m, mo);
    l = (m == -INFINITY ? 0.f : l * __expf(m - mn)) + (mo == -INFINITY ? 0.f : lo * __expf(mo - mn));
    m = mn;
  }
  if (lane == 0) {
    part[row] = make_float2(m, l);
    const int y = labels[row];
    if (y >= vlo && y < vlo + Vs && y < vocab) zlab[row] = zr[y - vlo];
  }
}

// single block: per row combine shards -> lse; loss sum in fixed order
__global__ __launch_bounds__(1024) void ce_combine_kernel(int rows, int n_shards, const float2* parts,
                                                          const float* zlab, const int32_t* labels,
                                                          int vocab, float* lse, float* loss,
                                                          float* inv_n) {
  __shared__ float s_loss[1024];
  __shared__ int s_cnt[1024];
  float acc = 0.f;
  int cnt = 0;
  // one row's lse from its shards' (max, sum) pairs; the loss sum in row order
  auto row_done = [&](int t, float m, float l, int y, float zl) __attribute__((always_inline)) {
    const float v = m + __logf(l);
    lse[t] = v;
    if (y >= 0 && y < vocab) {
      acc += v - zl;
      cnt += 1;
    }
  };
  constexpr int U = 8, MS = 4;  // rows per batch, shards held in registers
  if (n_shards <= MS) {
    // every load of U rows issued before the first use: the kernel is one
    // block, and one dependent load after another would set its time
    for (int t0 = threadIdx.x; t0 < rows; t0 += 1024 * U) {
      float2 pv[U][MS];
      int yv[U];
      float zv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + 1024 * u;
        const bool in = t < rows;
#pragma unroll
        for (int s = 0; s < MS; ++s)
          pv[u][s] = in && s < n_shards ? parts[(int64_t)s * rows + t] : make_float2(-INFINITY, 0.f);
        yv[u] = in ? labels[t] : -1;
        zv[u] = in ? zlab[t] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + 1024 * u;
        if (t >= rows) break;
        float m = -INFINITY;
#pragma unroll
        for (int s = 0; s < MS; ++s)
          if (s < n_shards) m = fmaxf(m, pv[u][s].x);
        float l = 0.f;
#pragma unroll
        for (int s = 0; s < MS; ++s)
          if (s < n_shards) l += pv[u][s].y * __expf(pv[u][s].x - m);
        row_done(t, m, l, yv[u], zv[u]);
      }
    }
  } else {
    for (int t = threadIdx.x; t < rows; t += 1024) {
      float m = -INFINITY;
      for (int s = 0; s < n_shards; ++s) m = fmaxf(m, parts[(int64_t)s * rows + t].x);
      float l = 0.f;
      for (int s = 0; s < n_shards; ++s) {
        const float2 p = parts[(int64_t)s * rows + t];
        l += p.y * __expf(p.x - m);
      }
      row_done(t, m, l, labels[t], zlab[t]);
    }
  }
  s_loss[threadIdx.x] = acc;
  s_cnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      s_loss[threadIdx.x] += s_loss[threadIdx.x + o];
      s_cnt[threadIdx.x] += s_cnt[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = s_cnt[0];
    loss[0] = n > 0 ? s_loss[0] / (float)n : 0.f;
    inv_n[0] = n > 0 ? 1.f / (float)n : 0.f;
  }
}

// one block per row: dz = (softmax(z) - onehot(label)) / n_valid for a
// labelled row, 0 for an ignored one. VEC: 16-byte loads and 4-element stores
// (row starts aligned), the ragged end one element per thread.
template <class T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  const uint32_t lo = uint32_t(to_bf16(a).u) | (uint32_t(to_bf16(b).u) << 16);
  const uint32_t hi = uint32_t(to_bf16(c).u) | (uint32_t(to_bf16(d).u) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

template <class T, bool VEC>
__global__ __launch_bounds__(256) void ce_grad_kernel(const float* __restrict__ z, int64_t ld, int Vs, int vlo,
                                                      const int32_t* __restrict__ labels, int vocab,
                                                      const float* __restrict__ lse, const float* __restrict__ inv_n,
                                                      T* __restrict__ dz, int64_t ldz) {
  const int t = blockIdx.x;
  const int y = labels[t];
  const bool valid = y >= 0 && y < vocab;
  const float lt = lse[t], sc = valid ? inv_n[0] : 0.f;
  const int yl = valid ? y - vlo : -1;  // label column within the shard (may lie outside it)
  const float* zr = z + (int64_t)t * ld;
  T* dr = dz + (int64_t)t * ldz;
  int c0 = 0;
  if constexpr (VEC) {
    const float4* z4 = reinterpret_cast<const float4*>(zr);
    const int n4 = Vs >> 2;
    auto emit = [&](int c, float4 v) __attribute__((always_inline)) {
      float o0 = __expf(v.x - lt) * sc, o1 = __expf(v.y - lt) * sc, o2 = __expf(v.z - lt) * sc,
            o3 = __expf(v.w - lt) * sc;
      const int j = yl - 4 * c;
      if (j == 0) o0 -= sc;
      if (j == 1) o1 -= sc;
      if (j == 2) o2 -= sc;
      if (j == 3) o3 -= sc;
      store4<T>(dr + 4 * c, o0, o1, o2, o3);
    };
    // four loads in flight per thread before the first result is stored
    int c = threadIdx.x;
    for (; c + 768 < n4; c += 1024) {
      const float4 a = z4[c], b = z4[c + 256], d = z4[c + 512], e = z4[c + 768];
      emit(c, a);
      emit(c + 256, b);
      emit(c + 512, d);
      emit(c + 768, e);
    }
    for (; c < n4; c += 256) emit(c, z4[c]);
    c0 = n4 << 2;
  }
  for (int c = c0 + threadIdx.x; c < Vs; c += 256) {
    float o = __expf(zr[c] - lt) * sc;
    if (c == yl) o -= sc;
    dr[c] = from_f<T>(o);
  }
}

// ---------------------------------------------------------------------------
// embedding
// ---------------------------------------------------------------------------
// an id outside [0, vocab) (e.g. a padding id of -100) gives a zero row, as
// the backward ignores it
template <class T>
__global__ void embed_fwd_kernel(const int32_t* ids, const T* table, T* x0, int rows, int vocab, int H) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * H) return;
  const int t = (int)(idx / H), c = (int)(idx % H);
  const int v = ids[t];
  x0[idx] = (v >= 0 && v < vocab) ? table[(int64_t)v * H + c] : from_f<T>(0.f);
}

// one block per vocabulary row, one thread per column: tokens scanned in order
template <class T>
__global__ void embed_bwd_kernel(const int32_t* ids, const T* dx0, float* dtable, int rows, int H) {
  const int v = blockIdx.x;
  for (int c = threadIdx.x; c < H; c += blockDim.x) {
    float s = 0.f;
    for (int t = 0; t < rows; ++t)
      if (ids[t] == v) s += to_f(dx0[(int64_t)t * H + c]);
    dtable[(int64_t)v * H + c] = s;
  }
}

// 64 x 64 tile per 256-thread block through LDS: 16-byte loads along the
// source rows, 16-byte stores along the destination rows
// dst[c][r] = src[r][c] over tiles of 128 source rows x 64 source columns.
// A thread loads the same 8 columns (16 bytes) of two adjacent source rows
// and pairs them column by column into 32-bit words, each two consecutive
// elements of one destination row; the tile is held destination-major as
// [64 rows][64 words] and written out 16 bytes per lane. The tile's 16-byte
// granules are XOR-swizzled by the destination row's group of 8, which
// spreads both the 4-byte stores (lanes of one store differ in column group
// and row pair) and the 16-byte reads (lanes differ in granule) over the
// banks. rows and cols are multiples of 8, so a 16-byte chunk is wholly in
// range or wholly out.
__device__ __forceinline__ int tr_word(int c, int w) { return c * 64 + (((w >> 2) ^ (c >> 3)) << 2) + (w & 3); }

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                             uint16_t* __restrict__ dst, int64_t ldd, int rows,
                                                             int cols) {
  __shared__ uint32_t tile[64 * 64];
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 64;
  const int q = threadIdx.x & 7;  // column group: source columns c0 + 8q .. + 7
  uint4 va[2], vb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w = (threadIdx.x >> 3) + 32 * h;  // word (row pair): source rows r0 + 2w, r0 + 2w + 1
    const int r = r0 + 2 * w, c = c0 + 8 * q;
    va[h] = vb[h] = make_uint4(0, 0, 0, 0);
    if (r < rows && c < cols) {
      va[h] = *reinterpret_cast<const uint4*>(src + (int64_t)r * lds + c);
      vb[h] = *reinterpret_cast<const uint4*>(src + (int64_t)(r + 1) * lds + c);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int w = (threadIdx.x >> 3) + 32 * h;
    const uint32_t a[4] = {va[h].x, va[h].y, va[h].z, va[h].w}, b[4] = {vb[h].x, vb[h].y, vb[h].z, vb[h].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // destination rows 8q + 2e (the low halves) and 8q + 2e + 1 (the high)
      tile[tr_word(8 * q + 2 * e, w)] = (a[e] & 0xffffu) | (b[e] << 16);
      tile[tr_word(8 * q + 2 * e + 1, w)] = (a[e] >> 16) | (b[e] & 0xffff0000u);
    }
  }
  __syncthreads();
  const int k = threadIdx.x & 15;  // granule: destination columns r0 + 8k .. + 7
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int c = (threadIdx.x >> 4) + 16 * h;  // destination row c0 + c
    if (c0 + c >= cols || r0 + 8 * k >= rows) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(&tile[tr_word(c, 4 * k)]);
    *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + c) * ldd + r0 + 8 * k) = v;
  }
}

__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N, float* __restrict__ C,
                                     int64_t ldc, int accumulate) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float v = 0.f;
  for (int sp = 0; sp < splits; ++sp) v += part[(int64_t)sp * M * N + idx];
  float* c = C + m * ldc + n;
  *c = accumulate ? *c + v : v;
}

template <class T>
__global__ void cast_kernel(const float* a, T* out, size_t n) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i < n) out[i] = from_f<T>(a[i]);
}

// fp32 -> bf16, four elements per thread (16-byte loads, 8-byte stores)
__global__ void cast4_bf16_kernel(const float4* __restrict__ a, uint2* __restrict__ out, size_t n4) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = a[i];
  out[i] = make_uint2((uint32_t)to_bf16(v.x).u | ((uint32_t)to_bf16(v.y).u << 16),
                      (uint32_t)to_bf16(v.z).u | ((uint32_t)to_bf16(v.w).u << 16));
}

unsigned blocks_for(int64_t n, int per = 256) { return (unsigned)cdiv(n, per); }

}  // namespace

rp_status fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return RP_OK;
  RP_CHECK(((uintptr_t)p & 15) == 0, RP_ERR_INVALID, "fill_zero: pointer not 16-byte aligned");
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  unsigned g = (unsigned)std::min<size_t>(std::max<size_t>(cdiv(n16, 256), 1), 8192);
  TraceScope ts(s, "fill_zero_kernel", 0.0, (double)bytes);
  RP_LAUNCH(fill_zero_kernel, dim3(g), dim3(256), 0, s, (uint4*)p, n16, (uint8_t*)p + n16 * 16, ntail);
  return RP_OK;
}

rp_status copy16(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes == 0) return RP_OK;
  RP_CHECK((((uintptr_t)dst | (uintptr_t)src | bytes) & 15) == 0, RP_ERR_INVALID,
           "copy: pointers and size must be multiples of 16 bytes");
  const size_t n16 = bytes / 16;
  unsigned g = (unsigned)std::min<size_t>(std::max<size_t>(cdiv(n16, 256), 1), 8192);
  TraceScope ts(s, "copy16_kernel", 0.0, 2.0 * bytes);
  RP_LAUNCH(copy16_kernel, dim3(g), dim3(256), 0, s, (uint4*)dst, (const uint4*)src, n16);
  return RP_OK;
}

rp_status convert_f32_bf16(void* dst, const void* src, size_t src_bytes, hipStream_t s) {
  if (src_bytes == 0) return RP_OK;
  RP_CHECK((((uintptr_t)dst | (uintptr_t)src) & 15) == 0 && src_bytes % 32 == 0, RP_ERR_INVALID,
           "bf16 conversion: 16-byte aligned ends and a multiple of 32 source bytes required");
  const size_t n8 = src_bytes / 32;
  TraceScope ts(s, "convert_f32_bf16_kernel", 0.0, 1.5 * (double)src_bytes);
  RP_LAUNCH(convert_f32_bf16_kernel, dim3((unsigned)std::min<size_t>((n8 + 255) / 256, 2048)), dim3(256), 0, s,
            (uint4*)dst, (const float4*)src, n8);
  return RP_OK;
}

rp_status rmsnorm_fwd(int dt, const void* x, const void* gamma, void* y, float* rstd, int T, int H,
                      float eps, hipStream_t s) {
  if (T == 0) return RP_OK;
  RP_CHECK(H % 8 == 0, RP_ERR_UNSUPPORTED, "rmsnorm: H %% 8 != 0");
  dim3 g(blocks_for(T, 4));
  const double bytes = (double)T * H * 2 * dtype_size(dt) + H * dtype_size(dt) + 4.0 * T;
  if (dt == RP_DTYPE_BF16 && H % 512 == 0) {
    auto rows = [&](auto nv_c) -> rp_status {
      constexpr int NV = decltype(nv_c)::value;
      TraceScope ts(s, "rmsnorm_fwd_rows_kernel", 0.0, bytes);
      RP_LAUNCH(rmsnorm_fwd_rows_kernel<NV>, g, dim3(256), 0, s, (const bf16*)x, (const bf16*)gamma, (bf16*)y,
                rstd, T, H, eps);
      return RP_OK;
    };
    switch (H / 512) {
      case 4: return rows(std::integral_constant<int, 4>{});
      case 8: return rows(std::integral_constant<int, 8>{});
      case 10: return rows(std::integral_constant<int, 10>{});
      case 16: return rows(std::integral_constant<int, 16>{});
      default: break;
    }
  }
  TraceScope ts(s, "rmsnorm_fwd_kernel", 0.0, bytes);
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(rmsnorm_fwd_kernel<bf16>, g, dim3(256), 0, s, (const bf16*)x, (const bf16*)gamma,
              (bf16*)y, rstd, T, H, eps);
  else
    RP_LAUNCH(rmsnorm_fwd_kernel<float>, g, dim3(256), 0, s, (const float*)x, (const float*)gamma,
              (float*)y, rstd, T, H, eps);
  return RP_OK;
}

rp_status sum_rows(const float* part, int nrow, int H, float* out, bool accumulate, hipStream_t s) {
  if (H == 0) return RP_OK;
  RP_LAUNCH(sum_rows_kernel, dim3((unsigned)cdiv(H, 32)), dim3(256), 0, s, part, nrow, H, out, (int)accumulate);
  return RP_OK;
}

size_t rmsnorm_bwd_part_bytes(int T, int H) {
  return (size_t)cdiv(T, RMS_BWD_ROWS) * H * sizeof(float);
}

template <class T, class TR, int NC>
static rp_status rows_bwd(const float* g, const void* x, const void* gamma, const float* rstd, const void* resid,
                          float* out_f32, void* out_dt, float* part, int rows, unsigned nb, size_t lds,
                          hipStream_t s) {
  if (lds > 32 * 1024)
    RP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rmsnorm_bwd_rows_kernel<T, TR, NC>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  RP_LAUNCH((rmsnorm_bwd_rows_kernel<T, TR, NC>), dim3(nb), dim3(256), lds, s, g, (const T*)x, (const T*)gamma, rstd,
            (const TR*)resid, out_f32, (T*)out_dt, part, rows);
  return RP_OK;
}

template <class T>
static rp_status rmsnorm_bwd_t(const float* g, const void* x, const void* gamma, const float* rstd,
                               const void* resid, int resid_dt, float* out_f32, void* out_dt,
                               float* dgamma, bool dgamma_acc, float* part, int rows, int H, hipStream_t s) {
  const unsigned nb = blocks_for(rows, RMS_BWD_ROWS);
  const size_t lds = 4 * (size_t)H * sizeof(float);
  constexpr int V = Vec<T>::N;
  const int nc = H % (64 * V) == 0 ? H / (64 * V) : 0;
  // g (fp32), x, out, resid read/written once; dgamma partials
  const double es = sizeof(T);
  TraceScope ts(s, "rmsnorm_bwd_kernel", 0.0,
                (double)rows * H * (4.0 + 2 * es + (resid ? (resid_dt == RP_DTYPE_F32 ? 4.0 : 2.0) : 0.0) +
                                    (out_f32 ? 4.0 : 0.0) - (out_dt ? 0.0 : es)) + 4.0 * rows);
  RP_CHECK(lds <= 160 * 1024, RP_ERR_UNSUPPORTED, "rmsnorm bwd: H too large");
  if (lds > 32 * 1024) {
    if (resid_dt == RP_DTYPE_F32)
      RP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rmsnorm_bwd_kernel<T, float>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    else
      RP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rmsnorm_bwd_kernel<T, bf16>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  }
  const bool rf32 = resid_dt == RP_DTYPE_F32 || resid == nullptr;
  if (nc == 1 || nc == 2 || nc == 4 || nc == 8) {
    // the row fits the registers of one wave (up to 4096 bf16 / 2048 fp32)
    RP_TRY(nc == 1   ? (rf32 ? rows_bwd<T, float, 1>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s)
                             : rows_bwd<T, bf16, 1>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s))
           : nc == 2 ? (rf32 ? rows_bwd<T, float, 2>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s)
                             : rows_bwd<T, bf16, 2>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s))
           : nc == 4 ? (rf32 ? rows_bwd<T, float, 4>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s)
                             : rows_bwd<T, bf16, 4>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s))
                     : (rf32 ? rows_bwd<T, float, 8>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s)
                             : rows_bwd<T, bf16, 8>(g, x, gamma, rstd, resid, out_f32, out_dt, part, rows, nb, lds, s)));
  } else if (rf32) {
    RP_LAUNCH((rmsnorm_bwd_kernel<T, float>), dim3(nb), dim3(256), lds, s, g, (const T*)x,
              (const T*)gamma, rstd, (const float*)resid, out_f32, (T*)out_dt, part, rows, H);
  } else {
    RP_LAUNCH((rmsnorm_bwd_kernel<T, bf16>), dim3(nb), dim3(256), lds, s, g, (const T*)x,
              (const T*)gamma, rstd, (const bf16*)resid, out_f32, (T*)out_dt, part, rows, H);
  }
  if (dgamma)
    RP_LAUNCH(sum_rows_kernel, dim3((unsigned)cdiv(H, 32)), dim3(256), 0, s, part, (int)nb, H, dgamma, (int)dgamma_acc);
  return RP_OK;
}

rp_status rmsnorm_bwd(int dt, const float* g, const void* x, const void* gamma, const float* rstd,
                      const void* resid, int resid_dt, float* out_f32, void* out_dt, float* dgamma,
                      bool dgamma_acc, float* part, int T, int H, hipStream_t s) {
  if (T == 0) {
    if (dgamma && !dgamma_acc) return fill_zero(dgamma, (size_t)H * 4, s);
    return RP_OK;
  }
  RP_CHECK(H % 8 == 0, RP_ERR_UNSUPPORTED, "rmsnorm: H %% 8 != 0");
  if (dt == RP_DTYPE_BF16)
    return rmsnorm_bwd_t<bf16>(g, x, gamma, rstd, resid, resid_dt, out_f32, out_dt, dgamma, dgamma_acc, part, T, H,
                               s);
  return rmsnorm_bwd_t<float>(g, x, gamma, rstd, resid, resid_dt, out_f32, out_dt, dgamma, dgamma_acc, part, T, H,
                              s);
}

rp_status rope_table(float2* tab, int seq, int d, float base, hipStream_t s) {
  const int64_t n = (int64_t)seq * (d / 2);
  if (n == 0) return RP_OK;
  RP_LAUNCH(rope_table_kernel, dim3(blocks_for(n)), dim3(256), 0, s, tab, seq, d, (double)base);
  return RP_OK;
}

rp_status rope_apply(int dt, void* buf, int64_t ld, int T, int seq, int n_heads, int d,
                     const float2* tab, bool inverse, hipStream_t s) {
  const int64_t n = (int64_t)T * n_heads * (d / 2);
  if (n == 0) return RP_OK;
  const bool v4 =
      dt == RP_DTYPE_BF16 && d % 8 == 0 && ld % 4 == 0 && ((uintptr_t)buf & 7) == 0 && ((uintptr_t)tab & 15) == 0;
  TraceScope ts(s, v4 ? "rope_apply4_kernel" : "rope_apply_kernel", 0.0, (double)n * 4 * dtype_size(dt));
  if (v4)
    RP_LAUNCH(rope_apply4_kernel, dim3(blocks_for(n / 4)), dim3(256), 0, s, (bf16*)buf, ld, T, seq, n_heads, d, tab,
              inverse ? 1 : 0);
  else if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(rope_apply_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, s, (bf16*)buf, ld, T, seq,
              n_heads, d, tab, inverse ? 1 : 0);
  else
    RP_LAUNCH(rope_apply_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, s, (float*)buf, ld, T, seq,
              n_heads, d, tab, inverse ? 1 : 0);
  return RP_OK;
}

rp_status swiglu_fwd(int dt, const void* gu, void* m, int T, int F, hipStream_t s) {
  const int64_t n = (int64_t)T * F;
  if (n == 0) return RP_OK;
  TraceScope ts(s, "swiglu_fwd_kernel", 0.0, (double)n * 3 * dtype_size(dt));
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(swiglu_fwd_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, s, (const bf16*)gu, (bf16*)m, T, F);
  else
    RP_LAUNCH(swiglu_fwd_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, s, (const float*)gu, (float*)m, T, F);
  return RP_OK;
}

rp_status swiglu_bwd(int dt, const float* dm, const void* gu, void* dgu, int T, int F, hipStream_t s) {
  const int64_t n = (int64_t)T * F;
  if (n == 0) return RP_OK;
  TraceScope ts(s, "swiglu_bwd_kernel", 0.0, (double)n * (4 + 4 * dtype_size(dt)));
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(swiglu_bwd_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, s, dm, (const bf16*)gu, (bf16*)dgu, T, F);
  else
    RP_LAUNCH(swiglu_bwd_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, s, dm, (const float*)gu, (float*)dgu, T, F);
  return RP_OK;
}

rp_status ce_shard_stats(const float* logits, int64_t ld, int T, int Vs, int vlo, const int32_t* labels,
                         int vocab, float2* part, float* zlab, hipStream_t s) {
  if (T == 0) return RP_OK;
  TraceScope ts(s, "ce_stats_kernel", 0.0, (double)T * Vs * 4 + 16.0 * T);
  if (((uintptr_t)logits & 15) == 0 && ld % 4 == 0)
    RP_LAUNCH(ce_stats_kernel<true>, dim3(blocks_for(T, 4)), dim3(256), 0, s, logits, ld, T, Vs, vlo, labels,
              vocab, part, zlab);
  else
    RP_LAUNCH(ce_stats_kernel<false>, dim3(blocks_for(T, 4)), dim3(256), 0, s, logits, ld, T, Vs, vlo, labels,
              vocab, part, zlab);
  return RP_OK;
}

rp_status ce_combine(int T, int n_shards, const float2* parts, const float* zlab, const int32_t* labels,
                     int vocab, float* lse, float* loss, float* inv_n, hipStream_t s) {
  TraceScope ts(s, "ce_combine_kernel", 0.0, (double)T * (8.0 * n_shards + 12.0));
  RP_LAUNCH(ce_combine_kernel, dim3(1), dim3(1024), 0, s, T, n_shards, parts, zlab, labels, vocab, lse,
            loss, inv_n);
  return RP_OK;
}

rp_status ce_grad(int dt, const float* logits, int64_t ld, int T, int Vs, int vlo, const int32_t* labels,
                  int vocab, const float* lse, const float* inv_n, void* dz, int64_t ldz, hipStream_t s) {
  const int64_t n = (int64_t)T * Vs;
  if (n == 0) return RP_OK;
  TraceScope ts(s, "ce_grad_kernel", 0.0, (double)n * (4 + dtype_size(dt)) + 8.0 * T);
  const size_t es = dtype_size(dt);
  const bool vec = ((uintptr_t)logits & 15) == 0 && ld % 4 == 0 && ((uintptr_t)dz & (4 * es - 1)) == 0 && ldz % 4 == 0;
  const dim3 g((unsigned)T), b(256);
  if (dt == RP_DTYPE_BF16) {
    if (vec)
      RP_LAUNCH((ce_grad_kernel<bf16, true>), g, b, 0, s, logits, ld, Vs, vlo, labels, vocab, lse, inv_n, (bf16*)dz, ldz);
    else
      RP_LAUNCH((ce_grad_kernel<bf16, false>), g, b, 0, s, logits, ld, Vs, vlo, labels, vocab, lse, inv_n, (bf16*)dz, ldz);
  } else {
    if (vec)
      RP_LAUNCH((ce_grad_kernel<float, true>), g, b, 0, s, logits, ld, Vs, vlo, labels, vocab, lse, inv_n, (float*)dz, ldz);
    else
      RP_LAUNCH((ce_grad_kernel<float, false>), g, b, 0, s, logits, ld, Vs, vlo, labels, vocab, lse, inv_n, (float*)dz, ldz);
  }
  return RP_OK;
}

rp_status embed_fwd(int dt, const int32_t* ids, const void* table, void* x0, int T, int V, int H,
                    hipStream_t s) {
  const int64_t n = (int64_t)T * H;
  if (n == 0) return RP_OK;
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(embed_fwd_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, s, ids, (const bf16*)table, (bf16*)x0, T, V,
              H);
  else
    RP_LAUNCH(embed_fwd_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, s, ids, (const float*)table, (float*)x0, T,
              V, H);
  return RP_OK;
}

rp_status embed_bwd(int dt, const int32_t* ids, const void* dx0, float* dtable, int T, int V, int H,
                    hipStream_t s) {
  if (V == 0) return RP_OK;
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(embed_bwd_kernel<bf16>, dim3(V), dim3(256), 0, s, ids, (const bf16*)dx0, dtable, T, H);
  else
    RP_LAUNCH(embed_bwd_kernel<float>, dim3(V), dim3(256), 0, s, ids, (const float*)dx0, dtable, T, H);
  return RP_OK;
}

rp_status transpose_bf16(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return RP_OK;
  RP_CHECK(rows % 8 == 0 && cols % 8 == 0 && lds % 8 == 0 && ldd % 8 == 0 && ((uintptr_t)src & 15) == 0 &&
               ((uintptr_t)dst & 15) == 0,
           RP_ERR_UNSUPPORTED, "transpose: sizes and leading dimensions must be multiples of 8, 16-byte aligned");
  TraceScope ts(s, "transpose_bf16_kernel", 0.0, 4.0 * rows * cols);
  RP_LAUNCH(transpose_bf16_kernel, dim3((unsigned)cdiv(cols, 64), (unsigned)cdiv(rows, 128)), dim3(256), 0, s,
            (const uint16_t*)src, lds, (uint16_t*)dst, ldd, rows, cols);
  return RP_OK;
}

rp_status splitk_reduce(const float* part, int splits, int M, int N, float* C, int64_t ldc, bool accumulate,
                        hipStream_t s) {
  const int64_t n = (int64_t)M * N;
  if (n == 0) return RP_OK;
  TraceScope ts(s, "splitk_reduce_kernel", 0.0, (double)n * 4 * (splits + 1 + (accumulate ? 1 : 0)));
  RP_LAUNCH(splitk_reduce_kernel, dim3(blocks_for(n)), dim3(256), 0, s, part, splits, M, N, C, ldc, accumulate ? 1 : 0);
  return RP_OK;
}

rp_status cast_from_f32(int dt, const float* a, void* out, size_t n, hipStream_t s) {
  if (n == 0) return RP_OK;
  const bool v4 = dt == RP_DTYPE_BF16 && n % 4 == 0 && ((uintptr_t)a & 15) == 0 && ((uintptr_t)out & 7) == 0;
  TraceScope ts(s, v4 ? "cast4_bf16_kernel" : "cast_kernel", 0.0, (double)n * (4 + dtype_size(dt)));
  if (v4)
    RP_LAUNCH(cast4_bf16_kernel, dim3(blocks_for((int64_t)(n / 4))), dim3(256), 0, s, (const float4*)a, (uint2*)out,
              n / 4);
  else if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(cast_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, s, a, (bf16*)out, n);
  else
    RP_LAUNCH(cast_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, s, a, (float*)out, n);
  return RP_OK;
}

}  // namespace rp
