// Causal GQA attention of the decoder layer, forward and backward, on a packed
// qkv buffer [T, (n_q + 2 n_kv) d] (q and k already rotated by RoPE).
// Query head h reads kv head floor(h * n_kv / n_q); scores are scaled by
// 1/sqrt(d); the causal mask keeps keys at positions <= the query's, within
// the query's own batch row. The forward also stores lse = log-sum-exp of the
// scaled scores per (head, token), which the backward uses to rebuild the
// probabilities without storing them (flash-attention style; the paper's
// appendix B.1 assumes FlashAttention for the stored attention state).
//
// This file holds the reference-grade kernels (one wavefront per query row,
// lanes over the head dimension), used for fp32 and for head_dim 64, and the
// MFMA flash kernels for bf16 with head_dim 128 (attn_flash.hip).
#include <mutex>
#include <vector>

#include "ops.h"
#include "attn_flash.h"
#include "trace.h"

namespace rp {
namespace {

// The allocation-free backward's per-row softmax terms D = rowsum(dO * O):
// one fixed array per GPU, held until the process ends. In host code this
// name is a host-side stand-in, never a device address: kernels get the
// address that attn_scratch() looked up for the device.
static __device__ __align__(256) float scratch[kAttnScratchFloats];

// causal (query, key) pairs of all batch rows
double causal_pairs(const AttnDesc& a) { return (double)a.batch * a.seq * (a.seq + 1.0) / 2.0; }

template <class T, int DPL>  // DPL = head_dim / 64 elements per lane
__global__ __launch_bounds__(256) void attn_fwd_simple(const T* __restrict__ qkv, T* __restrict__ o,
                                                       float* __restrict__ lse, int T_, int seq, int nq,
                                                       int nkv, float scale) {
  constexpr int D = DPL * 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)T_ * nq) return;
  const int t = (int)(w / nq), h = (int)(w % nq);
  const int hk = (h * nkv) / nq;
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int row0 = (t / seq) * seq;
  float q[DPL], acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    q[i] = to_f(qkv[(int64_t)t * ld + h * D + lane + 64 * i]) * scale;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int u = row0; u <= t; ++u) {
    const T* kr = qkv + (int64_t)u * ld + (int64_t)(nq + hk) * D;
    const T* vr = qkv + (int64_t)u * ld + (int64_t)(nq + nkv + hk) * D;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) s = fmaf(q[i], to_f(kr[lane + 64 * i]), s);
    s = wave_sum(s);
    const float mn = fmaxf(m, s);
    const float c = __expf(m - mn), p = __expf(s - mn);
    l = l * c + p;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = acc[i] * c + p * to_f(vr[lane + 64 * i]);
    m = mn;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[(int64_t)t * nq * D + h * D + lane + 64 * i] = from_f<T>(acc[i] * inv);
  if (lane == 0) lse[(int64_t)h * T_ + t] = m + __logf(l);
}

// dq for one (t, h) per wave; also writes D[h][t] = dO . O
template <class T, int DPL>
__global__ __launch_bounds__(256) void attn_dq_simple(const T* __restrict__ qkv, const T* __restrict__ o,
                                                      const T* __restrict__ dout, const float* __restrict__ lse,
                                                      float* __restrict__ Dbuf, T* __restrict__ dqkv, int T_,
                                                      int seq, int nq, int nkv, float scale) {
  constexpr int D = DPL * 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)T_ * nq) return;
  const int t = (int)(w / nq), h = (int)(w % nq);
  const int hk = (h * nkv) / nq;
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int row0 = (t / seq) * seq;
  float q[DPL], dov[DPL], dq[DPL];
  float dd = 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int64_t oi = (int64_t)t * nq * D + h * D + lane + 64 * i;
    q[i] = to_f(qkv[(int64_t)t * ld + h * D + lane + 64 * i]);
    dov[i] = to_f(dout[oi]);
    dd = fmaf(dov[i], to_f(o[oi]), dd);
    dq[i] = 0.f;
  }
  dd = wave_sum(dd);
  if (lane == 0) Dbuf[(int64_t)h * T_ + t] = dd;
  const float L = lse[(int64_t)h * T_ + t];
  for (int u = row0; u <= t; ++u) {
    const T* kr = qkv + (int64_t)u * ld + (int64_t)(nq + hk) * D;
    const T* vr = qkv + (int64_t)u * ld + (int64_t)(nq + nkv + hk) * D;
    float s = 0.f, dp = 0.f;
    float kv[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      kv[i] = to_f(kr[lane + 64 * i]);
      s = fmaf(q[i], kv[i], s);
      dp = fmaf(dov[i], to_f(vr[lane + 64 * i]), dp);
    }
    s = wave_sum(s);
    dp = wave_sum(dp);
    const float p = __expf(s * scale - L);
    const float ds = p * (dp - dd);
#pragma unroll
    for (int i = 0; i < DPL; ++i) dq[i] = fmaf(ds, kv[i], dq[i]);
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) dqkv[(int64_t)t * ld + h * D + lane + 64 * i] = from_f<T>(dq[i] * scale);
}

// dk, dv for one (u, kv head) per wave, summed over the query heads of its group
template <class T, int DPL>
__global__ __launch_bounds__(256) void attn_dkdv_simple(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ Dbuf, T* __restrict__ dqkv,
                                                        int T_, int seq, int nq, int nkv, float scale) {
  constexpr int D = DPL * 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)T_ * nkv) return;
  const int u = (int)(w / nkv), hk = (int)(w % nkv);
  const int64_t ld = (int64_t)(nq + 2 * nkv) * D;
  const int row_end = (u / seq + 1) * seq;
  const int G = nq / nkv;
  float k[DPL], v[DPL], dk[DPL], dv[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    k[i] = to_f(qkv[(int64_t)u * ld + (int64_t)(nq + hk) * D + lane + 64 * i]);
    v[i] = to_f(qkv[(int64_t)u * ld + (int64_t)(nq + nkv + hk) * D + lane + 64 * i]);
    dk[i] = dv[i] = 0.f;
  }
  for (int h = hk * G; h < (hk + 1) * G; ++h) {
    for (int t = u; t < row_end; ++t) {
      const T* qr = qkv + (int64_t)t * ld + h * D;
      const T* dor = dout + (int64_t)t * nq * D + h * D;
      float s = 0.f, dp = 0.f, qv[DPL], dov[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        qv[i] = to_f(qr[lane + 64 * i]);
        dov[i] = to_f(dor[lane + 64 * i]);
        s = fmaf(qv[i], k[i], s);
        dp = fmaf(dov[i], v[i], dp);
      }
      s = wave_sum(s);
      dp = wave_sum(dp);
      const float p = __expf(s * scale - lse[(int64_t)h * T_ + t]);
      const float ds = p * (dp - Dbuf[(int64_t)h * T_ + t]);
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        dv[i] = fmaf(p, dov[i], dv[i]);
        dk[i] = fmaf(ds, qv[i], dk[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    dqkv[(int64_t)u * ld + (int64_t)(nq + hk) * D + lane + 64 * i] = from_f<T>(dk[i] * scale);
    dqkv[(int64_t)u * ld + (int64_t)(nq + nkv + hk) * D + lane + 64 * i] = from_f<T>(dv[i]);
  }
}

template <class T, int DPL>
rp_status fwd_simple(const AttnDesc& a, const void* qkv, void* o, float* lse, hipStream_t s) {
  const int T_ = a.batch * a.seq;
  const int64_t waves = (int64_t)T_ * a.n_q;
  const float scale = 1.0f / sqrtf((float)a.d);
  TraceScope ts(s, "attn_fwd_simple", 4.0 * a.d * a.n_q * causal_pairs(a), 0.0);
  RP_LAUNCH((attn_fwd_simple<T, DPL>), dim3((unsigned)cdiv(waves, 4)), dim3(256), 0, s, (const T*)qkv, (T*)o,
            lse, T_, a.seq, a.n_q, a.n_kv, scale);
  return RP_OK;
}

template <class T, int DPL>
rp_status bwd_simple(const AttnDesc& a, const void* qkv, const void* o, const void* dout, const float* lse,
                     float* Dbuf, void* dqkv, hipStream_t s) {
  const int T_ = a.batch * a.seq;
  const float scale = 1.0f / sqrtf((float)a.d);
  TraceScope ts(s, "attn_bwd_simple", 8.0 * a.d * a.n_q * causal_pairs(a), 0.0);
  RP_LAUNCH((attn_dq_simple<T, DPL>), dim3((unsigned)cdiv((int64_t)T_ * a.n_q, 4)), dim3(256), 0, s,
            (const T*)qkv, (const T*)o, (const T*)dout, lse, Dbuf, (T*)dqkv, T_, a.seq, a.n_q, a.n_kv, scale);
  RP_LAUNCH((attn_dkdv_simple<T, DPL>), dim3((unsigned)cdiv((int64_t)T_ * a.n_kv, 4)), dim3(256), 0, s,
            (const T*)qkv, (const T*)dout, lse, Dbuf, (T*)dqkv, T_, a.seq, a.n_q, a.n_kv, scale);
  return RP_OK;
}

rp_status check(const AttnDesc& a) {
  RP_CHECK(a.d == 64 || a.d == 128, RP_ERR_UNSUPPORTED, "attention: head_dim must be 64 or 128");
  RP_CHECK(a.n_kv > 0 && a.n_q % a.n_kv == 0, RP_ERR_UNSUPPORTED, "attention: n_q %% n_kv != 0");
  RP_CHECK(a.batch >= 0 && a.seq >= 0, RP_ERR_INVALID, "attention: negative size");
  return RP_OK;
}

}  // namespace

rp_status attn_fwd(const AttnDesc& a, const void* qkv, void* o, float* lse, hipStream_t s) {
  RP_TRY(check(a));
  if (a.batch * a.seq == 0) return RP_OK;
  if (a.dt == RP_DTYPE_BF16 && a.d == 128 && flash_supported(a)) return flash_fwd(a, qkv, o, lse, s);
  if (a.dt == RP_DTYPE_BF16)
    return a.d == 128 ? fwd_simple<bf16, 2>(a, qkv, o, lse, s) : fwd_simple<bf16, 1>(a, qkv, o, lse, s);
  return a.d == 128 ? fwd_simple<float, 2>(a, qkv, o, lse, s) : fwd_simple<float, 1>(a, qkv, o, lse, s);
}

bool attn_bwd_fuses_rope(const AttnDesc& a) { return a.dt == RP_DTYPE_BF16 && a.d == 128 && flash_supported(a); }

rp_status attn_bwd(const AttnDesc& a, const void* qkv, const void* o, const void* dout, const float* lse,
                   float* Dbuf, void* dqkv, hipStream_t s, const float2* rope_inv) {
  RP_TRY(check(a));
  RP_CHECK(!rope_inv || attn_bwd_fuses_rope(a), RP_ERR_UNSUPPORTED, "attn_bwd: no fused rotation for this shape");
  if (a.batch * a.seq == 0) return RP_OK;
  if (attn_bwd_fuses_rope(a)) return flash_bwd(a, qkv, o, dout, lse, Dbuf, dqkv, s, rope_inv);
  if (a.dt == RP_DTYPE_BF16)
    return a.d == 128 ? bwd_simple<bf16, 2>(a, qkv, o, dout, lse, Dbuf, dqkv, s)
                      : bwd_simple<bf16, 1>(a, qkv, o, dout, lse, Dbuf, dqkv, s);
  return a.d == 128 ? bwd_simple<float, 2>(a, qkv, o, dout, lse, Dbuf, dqkv, s)
                    : bwd_simple<float, 1>(a, qkv, o, dout, lse, Dbuf, dqkv, s);
}

size_t attn_bwd_ws_bytes(const AttnDesc& a) { return (size_t)a.n_q * a.batch * a.seq * sizeof(float); }

rp_status attn_scratch(int device, float** out) {
  static std::mutex mu;
  static std::vector<float*> addr;  // per device, looked up once with that device current
  std::lock_guard<std::mutex> lock(mu);
  if (device < 0) {
    set_error("attention scratch: bad device %d", device);
    return RP_ERR_INVALID;
  }
  if ((size_t)device >= addr.size()) addr.resize(device + 1, nullptr);
  if (!addr[device]) {
    int cur = 0;
    RP_HIP(hipGetDevice(&cur));
    RP_CHECK(cur == device, RP_ERR_STATE, "attention scratch: device %d is not current (%d is)", device, cur);
    void* p = nullptr;
    RP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    RP_CHECK(p != nullptr, RP_ERR_HIP, "attention scratch: no device address");
    addr[device] = (float*)p;
  }
  *out = addr[device];
  return RP_OK;
}

}  // namespace rp
