// Internal launchers of the stage kernels (not part of the C ABI).
#pragma once

#include "common.h"

namespace rp {

// ---------------------------------------------------------------------------
// GEMM: C[M, N] = sum_k A(m, k) * B(n, k), fp32 accumulation
// ---------------------------------------------------------------------------
enum Epi {
  EPI_STORE = 0,      // C = acc (out dtype), or C += acc (fp32, accumulate)
  EPI_RESID = 1,      // C = acc + R (out dtype; R same dtype as C)
  EPI_SWIGLU = 2,     // B rows [0,F) gate, [F,2F) up: C = gu [M, 2F] pre-activations,
                      // C2 = silu(g) * u [M, F]; N passed = 2F
  EPI_SWIGLU_BWD = 3, // acc = dm [M, F]; R = gu [M, 2F]; C = dgu [M, 2F]
  EPI_ROPE = 4        // the packed q|k|v product with RoPE: columns are heads of
                      // 128; an optional R (same layout, bf16) is added, then
                      // heads < rope_heads are rotated (pairs i, i + 64 by the
                      // angle of position m % rope_seq) before the one bf16
                      // rounding; the others are stored as they are
};

// Grouped product: one GEMM per expert over that expert's rows, in one launch.
// Row tiles of GROUP_BM rows are mapped to (expert, first row) by tile_e /
// tile_m0 (built on the device from the routing); idle tiles have expert -1.
constexpr int GROUP_BM = 256;
struct GemmGroup {
  const int* tile_e = nullptr;
  const int* tile_m0 = nullptr;
  const int* off = nullptr;     // [E] first grouped row of each expert
  const int* cnt = nullptr;     // [E] rows of each expert
  const int* rows = nullptr;    // gathered A: operand row of each grouped row (null: A is grouped rows)
  int max_tiles_m = 0;          // size of the tile map
  int64_t a_rows = 0;           // rows of the A operand buffer
  int64_t b_stride = 0;         // elements between consecutive experts' B (N x K each)
};

struct GemmDesc {
  int M = 0, N = 0, K = 0;
  const void* A = nullptr; int64_t lda = 0; bool a_kmajor = true;
  const void* B = nullptr; int64_t ldb = 0; bool b_kmajor = true;
  void* C = nullptr; int64_t ldc = 0;
  int in_dtype = RP_DTYPE_BF16;   // A and B
  int out_dtype = RP_DTYPE_BF16;  // C (and C2, R)
  int epi = EPI_STORE;
  bool accumulate = false;
  const void* R = nullptr; int64_t ldr = 0;
  void* C2 = nullptr; int64_t ldc2 = 0;
  // EPI_SWIGLU: the caller reads only C2 afterwards, so the fused path does
  // not store the pre-activations into C (the unfused path still uses C as
  // its scratch)
  bool c_unused = false;
  float* tmp = nullptr;           // fp32 [M, N] scratch for the unfused fp32 path
  bool force_simple = false;      // use the generic kernel even for bf16
  float alpha = 1.f;              // C = alpha * A B^T (+ R): store / residual epilogues
  // split-K (bf16 operands, plain fp32 store): K is cut into split_k ranges,
  // each writes an fp32 partial into `partial` (splitk_bytes), and a fixed-
  // order reduction sums them into C (adding to C with accumulate).
  // split_k == 0: chosen from the tile count when `partial` is given
  int split_k = 1;
  float* partial = nullptr; size_t partial_bytes = 0;
  const float* row_scale = nullptr;  // per-row factor applied in the epilogue (grouped rows)
  const float2* rope_tab = nullptr;  // EPI_ROPE: (cos, sin) [rope_seq][64]
  int rope_seq = 0, rope_heads = 0;
  const GemmGroup* group = nullptr;  // gemm_grouped only
};

// grouped product over experts (see GemmGroup): M = total grouped rows (for
// accounting), N x K = one expert's B; C (and C2 / R) have one row per grouped
// row. Supported: SwiGLU and plain-store forwards (K-major B), SwiGLU-backward
// and plain-store input gradients (M-major B).
rp_status gemm_grouped(const GemmDesc& d, hipStream_t s);

size_t splitk_bytes(int64_t M, int64_t N, int64_t K, int split_k);
// C[m, n] (+)= sum over s < splits of part[s][m][n], in split order
rp_status splitk_reduce(const float* part, int splits, int M, int N, float* C, int64_t ldc, bool accumulate,
                        hipStream_t s);

rp_status gemm(const GemmDesc& d, hipStream_t s);
rp_status gemm_validate(const GemmDesc& d);

// ---------------------------------------------------------------------------
// elementwise / row kernels
// ---------------------------------------------------------------------------
rp_status fill_zero(void* p, size_t bytes, hipStream_t s);
rp_status copy16(void* dst, const void* src, size_t bytes, hipStream_t s);
// fp32 src (src_bytes) -> bf16 at dst (src_bytes / 2), round to nearest even
rp_status convert_f32_bf16(void* dst, const void* src, size_t src_bytes, hipStream_t s);

// y = x * rsqrt(mean(x^2) + eps) * gamma ; rstd[t] = rsqrt(...)
rp_status rmsnorm_fwd(int dt, const void* x, const void* gamma, void* y, float* rstd, int T,
                      int H, float eps, hipStream_t s);

// dx = (r * g*gamma - x * r^3 * mean(g*gamma*x)) + resid;  g fp32 [T, H].
// resid: nullptr, or [T, H] of dtype resid_dt. Writes out_f32 and/or out_dt.
// dgamma[h] = sum_t g[t,h] x[t,h] r[t] through part [n_part, H] partials
// (added to dgamma when dgamma_acc).
rp_status rmsnorm_bwd(int dt, const float* g, const void* x, const void* gamma,
                      const float* rstd, const void* resid, int resid_dt, float* out_f32,
                      void* out_dt, float* dgamma, bool dgamma_acc, float* part, int T, int H,
                      hipStream_t s);
size_t rmsnorm_bwd_part_bytes(int T, int H);
// column sums of part [nrow, H] into out[0 .. H) (added when accumulate)
rp_status sum_rows(const float* part, int nrow, int H, float* out, bool accumulate, hipStream_t s);

// QK-norm fused with RoPE on the q and k heads of qkv [T, ld] (in place):
// raw [T * (nq + nkv), d] keeps the pre-norm values, rstd [T * (nq + nkv)].
rp_status qknorm_rope_fwd(int dt, void* qkv, int64_t ld, void* raw, float* rstd, const void* gq, const void* gk,
                          int T, int seq, int nq, int nkv, int d, const float2* tab, float eps, hipStream_t s);
// Its backward, in place on the q and k heads of dqkv; dgamma (nullable) gets
// [gamma_q grad | gamma_k grad] (2d floats, added when dgamma_acc) through
// part (qknorm_part_bytes).
rp_status qknorm_rope_bwd(int dt, void* dqkv, int64_t ld, const void* raw, const float* rstd, const void* gq,
                          const void* gk, int T, int seq, int nq, int nkv, int d, const float2* tab, float* dgamma,
                          bool dgamma_acc, float* part, hipStream_t s);
size_t qknorm_part_bytes(int T, int n_heads, int d);

// cos/sin table [seq][d/2] (fp32 pairs) computed in fp64
rp_status rope_table(float2* tab, int seq, int d, float base, hipStream_t s);
// rotate (inverse=false) / rotate back (inverse=true) the first n_heads heads of
// every row of buf [T, ld] in place; position of row t is t % seq
rp_status rope_apply(int dt, void* buf, int64_t ld, int T, int seq, int n_heads, int d,
                     const float2* tab, bool inverse, hipStream_t s);

// m = silu(g) * u from gu [T, 2F]
rp_status swiglu_fwd(int dt, const void* gu, void* m, int T, int F, hipStream_t s);
// dgu from dm (fp32 [T, F]) and gu
rp_status swiglu_bwd(int dt, const float* dm, const void* gu, void* dgu, int T, int F,
                     hipStream_t s);

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
struct AttnDesc {
  int dt = RP_DTYPE_BF16;
  int batch = 1, seq = 0, n_q = 0, n_kv = 0, d = 0;
};
rp_status attn_fwd(const AttnDesc& a, const void* qkv, void* o, float* lse, hipStream_t s);
// Dbuf: fp32 [n_q, T] scratch. rope_inv (only where attn_bwd_fuses_rope):
// a RoPE table that dQ and dK are taken back through before they are stored
rp_status attn_bwd(const AttnDesc& a, const void* qkv, const void* o, const void* dout,
                   const float* lse, float* Dbuf, void* dqkv, hipStream_t s, const float2* rope_inv = nullptr);
bool attn_bwd_fuses_rope(const AttnDesc& a);
size_t attn_bwd_ws_bytes(const AttnDesc& a);
// the allocation-free backward's fixed scratch: kAttnScratchFloats fp32 per
// GPU (8 MiB: n_q * batch * seq <= 2^21); its device address for `device`,
// which must be current on the first call for that device
constexpr size_t kAttnScratchFloats = size_t(1) << 21;
rp_status attn_scratch(int device, float** out);

// ---------------------------------------------------------------------------
// cross-entropy over vocabulary shards
// ---------------------------------------------------------------------------
// per row of one shard's fp32 logits [T, Vs]: (max, sum exp(z - max)) -> part[t],
// and the label's logit into zlab[t] if the label falls in [vlo, vlo + Vs)
rp_status ce_shard_stats(const float* logits, int64_t ld, int T, int Vs, int vlo,
                         const int32_t* labels, int vocab, float2* part, float* zlab,
                         hipStream_t s);
// merge the shards' partials: lse[t]; loss = sum(lse - zlab) / n_valid; inv_n = 1/n_valid
rp_status ce_combine(int T, int n_shards, const float2* parts, const float* zlab,
                     const int32_t* labels, int vocab, float* lse, float* loss, float* inv_n,
                     hipStream_t s);
// dz = (exp(z - lse) - [v == label]) * inv_n (0 for ignored rows), dtype dt
rp_status ce_grad(int dt, const float* logits, int64_t ld, int T, int Vs, int vlo,
                  const int32_t* labels, int vocab, const float* lse, const float* inv_n,
                  void* dz, int64_t ldz, hipStream_t s);

// ---------------------------------------------------------------------------
// mixture of experts
// ---------------------------------------------------------------------------
// routing state of one MoE layer call (device buffers carved by the caller)
struct MoeRouting {
  int* idx = nullptr;       // [T, k] selected experts, descending logit
  float* wgt = nullptr;     // [T, k] softmax weights over the selected
  int* cnt = nullptr;       // [E] rows per expert
  int* off = nullptr;       // [E + 1] first grouped row per expert
  int* tile_e = nullptr;    // [max_tiles] tile map of the grouped products
  int* tile_m0 = nullptr;
  int max_tiles = 0;
  int* perm_row = nullptr;  // [T k] token of each grouped row
  float* perm_w = nullptr;  // [T k] routing weight of each grouped row
  int* inv = nullptr;       // [T k] grouped row of each (token, slot)
};
int moe_max_tiles(int64_t T, int k, int E);
// top-k routing, counting sort by expert, tile map
rp_status moe_route(const MoeRouting& m, const float* logits, int T, int E, int k, hipStream_t s);
// y = h1 + sum_s w * ye[row(t, s)]
rp_status moe_combine(const void* h1, const void* ye, const MoeRouting& m, int T, int k, int H, void* y,
                      hipStream_t s);
// db (fp32) = sum_s dbe[row(t, s)]
rp_status moe_uncombine(const void* dbe, const MoeRouting& m, int T, int k, int H, float* db, hipStream_t s);

// ---------------------------------------------------------------------------
// misc
// ---------------------------------------------------------------------------
rp_status embed_fwd(int dt, const int32_t* ids, const void* table, void* x0, int T, int V, int H,
                    hipStream_t s);
rp_status embed_bwd(int dt, const int32_t* ids, const void* dx0, float* dtable, int T, int V,
                    int H, hipStream_t s);
// dst [cols, rows] (leading dimension ldd) = src [rows, cols]^T (leading
// dimension lds), bf16; rows, cols, lds, ldd multiples of 8, 16-byte aligned
rp_status transpose_bf16(const void* src, int64_t lds, void* dst, int64_t ldd, int rows, int cols, hipStream_t s);
// out (dtype dt) = a (fp32)
rp_status cast_from_f32(int dt, const float* a, void* out, size_t n, hipStream_t s);

}  // namespace rp
