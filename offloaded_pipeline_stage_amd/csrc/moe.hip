// Mixture-of-experts routing and data movement of the MoE MLP (the layer of
// the paper's appendix C.2: every token runs its E_act selected experts out of
// E_total).
//
// route      per token: the k largest router logits (ties: lower expert
//            index) and their softmax weights over the selected k
// count/scan expert row counts, first rows, and the tile map of the grouped
//            products (GROUP_BM-row tiles -> (expert, first row))
// fill       the grouped order: the (token, slot) pairs of each expert in
//            increasing token then slot order (a stable counting sort), with
//            the inverse map (token, slot) -> grouped row
// combine    y[t] = h1[t] + sum over slots s of w[t, s] * ye[row(t, s)]
// uncombine  db[t] = sum over slots s of dbe[row(t, s)]
// Every kernel is deterministic: no atomics, sums in slot order.
#include "ops.h"
#include "trace.h"

namespace rp {
namespace {

constexpr int MAXE_PER_LANE = 4;  // up to 256 experts
constexpr int MAXK = 16;

// one wave per token
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        int* __restrict__ idx, float* __restrict__ wgt) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* z = logits + (int64_t)t * E;
  float v[MAXE_PER_LANE];
  bool taken[MAXE_PER_LANE];
#pragma unroll
  for (int j = 0; j < MAXE_PER_LANE; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? z[e] : -INFINITY;
    taken[j] = e >= E;
  }
  float sel_v[MAXK];
  int sel_e[MAXK];
  for (int s = 0; s < k; ++s) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < MAXE_PER_LANE; ++j) {
      const int e = lane + 64 * j;
      if (!taken[j] && (v[j] > bv || (v[j] == bv && e < be))) {
        bv = v[j];
        be = e;
      }
    }
    // (value descending, index ascending) over the wave, fixed butterfly order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    sel_v[s] = bv;
    sel_e[s] = be;
    if ((be & 63) == lane) {
#pragma unroll
      for (int j = 0; j < MAXE_PER_LANE; ++j)
        if (j == (be >> 6)) taken[j] = true;
    }
  }
  // softmax over the selected logits (the first is the largest)
  float den = 0.f;
  for (int s = 0; s < k; ++s) den += expf(sel_v[s] - sel_v[0]);
  for (int s = 0; s < k; ++s)
    if (lane == s) {
      idx[(int64_t)t * k + s] = sel_e[s];
      wgt[(int64_t)t * k + s] = expf(sel_v[s] - sel_v[0]) / den;
    }
}

// one block per expert: number of (token, slot) pairs routed to it
__global__ __launch_bounds__(256) void moe_count_kernel(const int* __restrict__ idx, int n, int* __restrict__ cnt) {
  __shared__ int part[4];
  const int e = blockIdx.x;
  int c = 0;
  for (int i = threadIdx.x; i < n; i += 256) c += idx[i] == e;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) cnt[e] = part[0] + part[1] + part[2] + part[3];
}

// single block: first rows and the tile map
__global__ __launch_bounds__(256) void moe_scan_kernel(const int* __restrict__ cnt, int E, int* __restrict__ off,
                                                       int* __restrict__ tile_e, int* __restrict__ tile_m0,
                                                       int max_tiles) {
  __shared__ int s_off[257], s_toff[257];
  if (threadIdx.x == 0) {
    s_off[0] = 0;
    s_toff[0] = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e + 1] = s_off[e] + cnt[e];
      s_toff[e + 1] = s_toff[e] + (cnt[e] + GROUP_BM - 1) / GROUP_BM;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += 256) off[e] = s_off[e];
  const int nt = s_toff[E];
  for (int i = threadIdx.x; i < max_tiles; i += 256) {
    int e = -1, m0 = 0;
    if (i < nt) {
      // the expert whose tile range holds i: largest e with s_toff[e] <= i
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_toff[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      e = lo;
      m0 = (i - s_toff[e]) * GROUP_BM;
    }
    tile_e[i] = e;
    tile_m0[i] = m0;
  }
}

// one block per expert: its pairs in (token, slot) order
__global__ __launch_bounds__(256) void moe_fill_kernel(const int* __restrict__ idx, const float* __restrict__ wgt,
                                                       int n, int k, const int* __restrict__ off,
                                                       int* __restrict__ perm_row, float* __restrict__ perm_w,
                                                       int* __restrict__ inv) {
  __shared__ int wtot[4];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int base = off[e];
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int i = c0 + threadIdx.x;
    const bool match = i < n && idx[i] == e;
    const unsigned long long bal = __ballot(match);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[w] = __popcll(bal);
    __syncthreads();
    int wbase = 0;
    for (int q = 0; q < w; ++q) wbase += wtot[q];
    const int total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
    if (match) {
      const int pos = base + wbase + before;
      perm_row[pos] = i / k;
      perm_w[pos] = wgt[i];
      inv[i] = pos;
    }
    base += total;
    __syncthreads();
  }
}

__device__ __forceinline__ void ld8(const bf16* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// one wave per token row, 8 columns per lane access
__global__ __launch_bounds__(256) void moe_combine_kernel(const bf16* __restrict__ h1, const bf16* __restrict__ ye,
                                                          const int* __restrict__ inv, const float* __restrict__ wgt,
                                                          int T, int k, int H, bf16* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  for (int c = lane * 8; c < H; c += 512) {
    float acc[8];
    ld8(h1 + (int64_t)t * H + c, acc);
    for (int s = 0; s < k; ++s) {
      const float wv = wgt[(int64_t)t * k + s];
      float r[8];
      ld8(ye + (int64_t)inv[(int64_t)t * k + s] * H + c, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wv, r[i], acc[i]);
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = uint32_t(to_bf16(acc[2 * i]).u) | (uint32_t(to_bf16(acc[2 * i + 1]).u) << 16);
    *reinterpret_cast<uint4*>(y + (int64_t)t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void moe_uncombine_kernel(const bf16* __restrict__ dbe, const int* __restrict__ inv,
                                                            int T, int k, int H, float* __restrict__ db) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  for (int c = lane * 8; c < H; c += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < k; ++s) {
      float r[8];
      ld8(dbe + (int64_t)inv[(int64_t)t * k + s] * H + c, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += r[i];
    }
    float* o = db + (int64_t)t * H + c;
    *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

int moe_max_tiles(int64_t T, int k, int E) { return (int)(cdiv(T * k, GROUP_BM) + E); }

rp_status moe_route(const MoeRouting& m, const float* logits, int T, int E, int k, hipStream_t s) {
  RP_CHECK(E >= k && k >= 1 && k <= MAXK && E <= 64 * MAXE_PER_LANE, RP_ERR_UNSUPPORTED,
           "moe: need 1 <= top_k <= %d, top_k <= experts <= %d", MAXK, 64 * MAXE_PER_LANE);
  RP_CHECK(logits != nullptr, RP_ERR_INVALID, "moe: router logits missing");
  const int n = T * k;
  {
    TraceScope ts(s, "moe_route_kernel", 0.0, (double)T * (E * 4.0 + k * 8.0));
    RP_LAUNCH(moe_route_kernel, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, s, logits, T, E, k, m.idx, m.wgt);
  }
  {
    TraceScope ts(s, "moe_count_kernel", 0.0, (double)E * n * 4.0);
    RP_LAUNCH(moe_count_kernel, dim3(E), dim3(256), 0, s, m.idx, n, m.cnt);
  }
  {
    TraceScope ts(s, "moe_scan_kernel", 0.0, (double)m.max_tiles * 8.0);
    RP_LAUNCH(moe_scan_kernel, dim3(1), dim3(256), 0, s, m.cnt, E, m.off, m.tile_e, m.tile_m0, m.max_tiles);
  }
  {
    TraceScope ts(s, "moe_fill_kernel", 0.0, (double)E * n * 4.0 + n * 16.0);
    RP_LAUNCH(moe_fill_kernel, dim3(E), dim3(256), 0, s, m.idx, m.wgt, n, k, m.off, m.perm_row, m.perm_w, m.inv);
  }
  return RP_OK;
}

rp_status moe_combine(const void* h1, const void* ye, const MoeRouting& m, int T, int k, int H, void* y,
                      hipStream_t s) {
  RP_CHECK(H % 8 == 0, RP_ERR_UNSUPPORTED, "moe combine: H %% 8 != 0");
  TraceScope ts(s, "moe_combine_kernel", 0.0, (double)T * H * 2 * (k + 2) + T * k * 8.0);
  RP_LAUNCH(moe_combine_kernel, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, s, (const bf16*)h1, (const bf16*)ye,
            m.inv, m.wgt, T, k, H, (bf16*)y);
  return RP_OK;
}

rp_status moe_uncombine(const void* dbe, const MoeRouting& m, int T, int k, int H, float* db, hipStream_t s) {
  RP_CHECK(H % 8 == 0, RP_ERR_UNSUPPORTED, "moe uncombine: H %% 8 != 0");
  TraceScope ts(s, "moe_uncombine_kernel", 0.0, (double)T * H * (2.0 * k + 4) + T * k * 4.0);
  RP_LAUNCH(moe_uncombine_kernel, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, s, (const bf16*)dbe, m.inv, T, k, H, db);
  return RP_OK;
}

}  // namespace rp
