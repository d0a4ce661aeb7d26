// Per-head RMSNorm of the query and key heads ahead of RoPE (the QK-norm of
// Qwen3-style layers), fused with the rotation: q_h <- R_p (gamma_q * q_h /
// sqrt(mean(q_h^2) + eps)), likewise k_h with gamma_k, on the packed qkv
// buffer in place. One lane holds one rotation pair (i, i + d/2) of a head,
// so a head spans d/2 lanes (64 for d = 128, 32 for d = 64) and its sum of
// squares is a reduction over those lanes.
#include <algorithm>

#include "ops.h"
#include "trace.h"

namespace rp {
namespace {

// forward: raw keeps the pre-norm values [rows * (nq + nkv), d] and rstd the
// per-(row, head) factor [rows * (nq + nkv)] for the backward
template <class T>
__global__ __launch_bounds__(256) void qknorm_rope_fwd_kernel(T* __restrict__ qkv, int64_t ld, T* __restrict__ raw,
                                                              float* __restrict__ rstd, const T* __restrict__ gq,
                                                              const T* __restrict__ gk, int rows, int seq, int nq,
                                                              int nkv, int d, const float2* __restrict__ tab,
                                                              float eps) {
  const int half = d / 2, hpw = 64 / half, nh = nq + nkv;
  const int lane = threadIdx.x & 63, i = lane % half;
  const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int64_t item = wave * hpw + lane / half;
  // a head's lanes leave together; the reductions below stay inside a head
  if (item >= (int64_t)rows * nh) return;
  const int row = (int)(item / nh), h = (int)(item % nh);
  T* base = qkv + (int64_t)row * ld + (int64_t)h * d;
  const T* gam = h < nq ? gq : gk;
  const T ra = base[i], rb = base[i + half];
  T* rw = raw + item * d;
  rw[i] = ra;
  rw[i + half] = rb;
  const float a = to_f(ra), b = to_f(rb);
  float ss = a * a + b * b;
  for (int o = half / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  const float na = a * r * to_f(gam[i]), nb = b * r * to_f(gam[i + half]);
  const float2 cs = tab[(int64_t)(row % seq) * half + i];
  base[i] = from_f<T>(na * cs.x - nb * cs.y);
  base[i + half] = from_f<T>(nb * cs.x + na * cs.y);
  if (i == 0) rstd[item] = r;
}

// backward, in place on the q and k heads of dqkv: rotate the gradient back
// (by -theta), then dx = r (g gamma) - x r^3 mean(g gamma x) per head; the
// gains' gradient sum_(row, head) g x r goes to part[block][0 .. 2d) (q heads,
// then k heads), each block summing its items in a fixed order
template <class T>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(T* __restrict__ dqkv, int64_t ld,
                                                              const T* __restrict__ raw,
                                                              const float* __restrict__ rstd,
                                                              const T* __restrict__ gq, const T* __restrict__ gk,
                                                              int rows, int seq, int nq, int nkv, int d,
                                                              const float2* __restrict__ tab, float* __restrict__ part) {
  __shared__ float red[4][2][128];
  const int half = d / 2, hpw = 64 / half, nh = nq + nkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, i = lane % half, grp = lane / half;
  const int64_t n_items = (int64_t)rows * nh;
  float aq0 = 0.f, aq1 = 0.f, ak0 = 0.f, ak1 = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 4 * hpw;
  for (int64_t first = ((int64_t)blockIdx.x * 4 + wave) * hpw; first < n_items; first += stride) {
    const int64_t item = first + grp;
    const bool valid = item < n_items;
    float ga = 0.f, gb = 0.f, xa = 0.f, xb = 0.f, r = 0.f, wa = 0.f, wb = 0.f;
    int h = 0;
    T* dp = nullptr;
    if (valid) {
      const int row = (int)(item / nh);
      h = (int)(item % nh);
      dp = dqkv + (int64_t)row * ld + (int64_t)h * d;
      const float2 cs = tab[(int64_t)(row % seq) * half + i];
      const float ya = to_f(dp[i]), yb = to_f(dp[i + half]);
      ga = ya * cs.x + yb * cs.y;
      gb = yb * cs.x - ya * cs.y;
      xa = to_f(raw[item * d + i]);
      xb = to_f(raw[item * d + i + half]);
      r = rstd[item];
      const T* gam = h < nq ? gq : gk;
      wa = to_f(gam[i]);
      wb = to_f(gam[i + half]);
    }
    float dot = ga * wa * xa + gb * wb * xb;
    for (int o = half / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
    if (valid) {
      const float c = r * r * r * dot / (float)d;
      dp[i] = from_f<T>(r * ga * wa - xa * c);
      dp[i + half] = from_f<T>(r * gb * wb - xb * c);
      if (h < nq) {
        aq0 += ga * xa * r;
        aq1 += gb * xb * r;
      } else {
        ak0 += ga * xa * r;
        ak1 += gb * xb * r;
      }
    }
  }
  if (part == nullptr) return;  // uniform over the block: no gain gradient wanted
  if (hpw == 2) {               // both heads of a wave hold the same elements
    aq0 += __shfl_xor(aq0, 32, 64);
    aq1 += __shfl_xor(aq1, 32, 64);
    ak0 += __shfl_xor(ak0, 32, 64);
    ak1 += __shfl_xor(ak1, 32, 64);
  }
  if (grp == 0) {
    red[wave][0][i] = aq0;
    red[wave][0][i + half] = aq1;
    red[wave][1][i] = ak0;
    red[wave][1][i + half] = ak1;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 2 * d; c += 256) {
    const int qk = c / d, e = c % d;
    part[(int64_t)blockIdx.x * 2 * d + c] = red[0][qk][e] + red[1][qk][e] + red[2][qk][e] + red[3][qk][e];
  }
}

}  // namespace

size_t qknorm_part_bytes(int T, int n_heads, int d) {
  const int hpw = 64 / (d / 2);
  const int64_t blocks = std::min<int64_t>(cdiv((int64_t)T * n_heads, 4 * hpw), 1024);
  return (size_t)std::max<int64_t>(blocks, 1) * 2 * d * sizeof(float);
}

rp_status qknorm_rope_fwd(int dt, void* qkv, int64_t ld, void* raw, float* rstd, const void* gq, const void* gk,
                          int T, int seq, int nq, int nkv, int d, const float2* tab, float eps, hipStream_t s) {
  RP_CHECK(d == 64 || d == 128, RP_ERR_UNSUPPORTED, "qk-norm: head_dim must be 64 or 128");
  const int64_t items = (int64_t)T * (nq + nkv);
  if (items == 0) return RP_OK;
  const int hpw = 64 / (d / 2);
  const unsigned blocks = (unsigned)cdiv(cdiv(items, hpw), 4);
  const double es = dtype_size(dt);
  TraceScope ts(s, "qknorm_rope_fwd_kernel", 0.0, (double)items * d * 3 * es + 4.0 * items);
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(qknorm_rope_fwd_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16*)qkv, ld, (bf16*)raw, rstd,
              (const bf16*)gq, (const bf16*)gk, T, seq, nq, nkv, d, tab, eps);
  else
    RP_LAUNCH(qknorm_rope_fwd_kernel<float>, dim3(blocks), dim3(256), 0, s, (float*)qkv, ld, (float*)raw, rstd,
              (const float*)gq, (const float*)gk, T, seq, nq, nkv, d, tab, eps);
  return RP_OK;
}

rp_status qknorm_rope_bwd(int dt, void* dqkv, int64_t ld, const void* raw, const float* rstd, const void* gq,
                          const void* gk, int T, int seq, int nq, int nkv, int d, const float2* tab, float* dgamma,
                          bool dgamma_acc, float* part, hipStream_t s) {
  RP_CHECK(d == 64 || d == 128, RP_ERR_UNSUPPORTED, "qk-norm: head_dim must be 64 or 128");
  const int64_t items = (int64_t)T * (nq + nkv);
  if (items == 0) {
    if (dgamma && !dgamma_acc) return fill_zero(dgamma, (size_t)2 * d * sizeof(float), s);
    return RP_OK;
  }
  const int hpw = 64 / (d / 2);
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(items, 4 * hpw), 1024);
  const double es = dtype_size(dt);
  TraceScope ts(s, "qknorm_rope_bwd_kernel", 0.0, (double)items * d * 3 * es + 4.0 * items);
  float* pp = dgamma ? part : nullptr;
  if (dt == RP_DTYPE_BF16)
    RP_LAUNCH(qknorm_rope_bwd_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16*)dqkv, ld, (const bf16*)raw, rstd,
              (const bf16*)gq, (const bf16*)gk, T, seq, nq, nkv, d, tab, pp);
  else
    RP_LAUNCH(qknorm_rope_bwd_kernel<float>, dim3(blocks), dim3(256), 0, s, (float*)dqkv, ld, (const float*)raw,
              rstd, (const float*)gq, (const float*)gk, T, seq, nq, nkv, d, tab, pp);
  if (dgamma) RP_TRY(sum_rows(part, (int)blocks, 2 * d, dgamma, dgamma_acc, s));
  return RP_OK;
}

}  // namespace rp
