// MFMA flash attention for bf16, head_dim 128 (forward and backward) on gfx950.
//
// Causal GQA attention of the decoder layer (query head h reads kv head
// floor(h * n_kv / n_q), scale 1/sqrt(d), keys at positions <= the query's
// within its own batch row), on the packed qkv buffer [T, (n_q + 2 n_kv) 128].
// The forward never materialises the scores: it streams 64-key tiles and keeps
// a running (max, sum) per query, and stores lse = log-sum-exp of the scaled
// scores so the backward can rebuild the probabilities (FlashAttention, which
// the paper's appendix B.1 assumes for the attention activations).
//
// Building block: v_mfma_f32_32x32x16_bf16. Operand A lane l holds row l%32,
// k = 8*(l/32)..+7; operand B lane l holds column l%32, the same k; the 32x32
// fp32 result lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4.
//
// Orientation: every product is arranged so that the 32 rows the wave owns
// (queries in the forward and dQ kernels, keys in the dK/dV kernel) are the
// MFMA *column* index, i.e. one row per lane. Then
//   - the softmax statistics of a query need only an in-lane reduction over
//     its 16 scores of a tile plus one exchange with lane l^32;
//   - a score tile (rows = streamed keys/queries held in registers) is the B
//     operand of the next product directly: the 16-element k-step j of a
//     32-row tile is registers 8j..8j+7, which hold rows 16j + {4h..4h+3,
//     8+4h..8+4h+3} for lane half h. The A operand read from LDS uses the same
//     row permutation, so the sum over k is unchanged.
// Streamed tiles (64 rows of K and V, or of Q and dO) go from global memory
// straight into LDS stages with buffer loads that target LDS, and are kept
// row-major only ([rows][128], 16-byte chunks XOR-swizzled by the row): the
// A operands of QK^T-type products are 16-byte fragment reads of it, those of
// PV-type products (the transposed tile) come from gfx950's transposing LDS
// read. No register staging and no in-register transposes; both read
// patterns are free of bank conflicts.
//
// The backward is two deterministic kernels (no atomics): dK/dV per key block
// (summing over the query heads of its kv group and all later queries), and
// dQ per query block; both recompute the probabilities from lse.
#include <type_traits>

#include "attn_flash.h"
#include "trace.h"

namespace rp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 128;        // head dim
constexpr int NT = 256;       // threads per workgroup (4 waves)
constexpr int WROWS = 32;     // rows owned by one wave
constexpr int BROWS = 128;    // rows owned by one workgroup
constexpr int TILE = 64;      // streamed rows per LDS tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_LOG2 = 8.f;  // forward: lazy rescale threshold (log2 units)

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float lane_of(float4 v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// wave index held in a scalar register, so that branches on the wave's rows
// (tile skipping, causal-mask tiles) are uniform branches, not masked code
__device__ __forceinline__ int wave_id(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Register-class hints for the one-wave-per-SIMD kernels, which use more
// than the 256 architectural registers: fragments that only ever feed MFMAs
// (the wave's own rows, held for the whole kernel) go to the accumulation
// registers, which MFMA operands may come from; score tiles, which the
// vector ALU reads next, to the architectural ones. Without them the
// compiler produced the score tiles in accumulation registers and copied
// them out for every tile.
__device__ __forceinline__ void to_acc_regs(bf16x8_t& f) { asm volatile("" : "+a"(f)); }
__device__ __forceinline__ void to_arch_regs(f32x16_t& t) { asm volatile("" : "+v"(t)); }

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// two fp32 values -> packed bf16 pair (round to nearest even), one
// v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// registers 8j..8j+7 of a score tile as a bf16x8 B operand
__device__ __forceinline__ bf16x8_t to_operand(const f32x16_t& c, int j) {
  u32x4_t u;
  u[0] = pack_bf16x2(c[8 * j + 0], c[8 * j + 1]);
  u[1] = pack_bf16x2(c[8 * j + 2], c[8 * j + 3]);
  u[2] = pack_bf16x2(c[8 * j + 4], c[8 * j + 5]);
  u[3] = pack_bf16x2(c[8 * j + 6], c[8 * j + 7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// B operand held in registers: row `row` (< rmax, else zero) of a strided
// matrix, columns [col, col + 128), d-step s for lane half h
__device__ __forceinline__ void load_rows_b(bf16x8_t (&f)[8], const bf16* g, int64_t ld, int row, int rmax, int col,
                                            int h) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (row < rmax) v = *reinterpret_cast<const u32x4_t*>(g + (int64_t)row * ld + col + 16 * s + 8 * h);
    f[s] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// store a [128 d x 32 rows] accumulator (rows on lanes) scaled by `mul` into
// row `row` of a strided bf16 matrix at column col. With `rot` (a RoPE table,
// (cos, sin) of position p and pair i at rot[64 p + i]) the values are first
// taken back through the rotation of the row's position: the gradient of the
// rotate-half pair (d, d + 64) is (a cos + b sin, b cos - a sin). A lane
// holds both members of its pairs (d-tiles dt and dt + 2), so this needs no
// exchange, and each value is rounded to bf16 once.
__device__ __forceinline__ void store_acc_rows(const f32x16_t (&acc)[4], float mul, bf16* g, int64_t ld, int row,
                                               int rmax, int col, int h, const float2* rot = nullptr) {
  if (row >= rmax) return;
  bf16* out = g + (int64_t)row * ld + col;
  float v[4][16];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[dt][r] = acc[dt][r] * mul;
  if (rot) {
    const float2* tr = rot + (int64_t)row * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // pairs 32 dt + 8 q + 4 h + e, e = 0..3: two 16-byte table reads
        const float4 t01 = *reinterpret_cast<const float4*>(tr + 32 * dt + 8 * q + 4 * h);
        const float4 t23 = *reinterpret_cast<const float4*>(tr + 32 * dt + 8 * q + 4 * h + 2);
        const float c[4] = {t01.x, t01.z, t23.x, t23.z}, sn[4] = {t01.y, t01.w, t23.y, t23.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = v[dt][4 * q + e], b = v[dt + 2][4 * q + e];
          v[dt][4 * q + e] = a * c[e] + b * sn[e];
          v[dt + 2][4 * q + e] = b * c[e] - a * sn[e];
        }
      }
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dt + 8 * q + 4 * h;
      u32x2_t u;
      u[0] = pack_bf16x2(v[dt][4 * q + 0], v[dt][4 * q + 1]);
      u[1] = pack_bf16x2(v[dt][4 * q + 2], v[dt][4 * q + 3]);
      *reinterpret_cast<u32x2_t*>(out + d) = u;
    }
}

struct FlashParams {
  const bf16* qkv;   // [T, ld]
  int64_t ld;        // (n_q + 2 n_kv) * 128
  int seq, nq, nkv;
  float c2;          // scale * log2(e)
  float scale;
  int n_blocks;      // row blocks of 128 per sequence
  const float2* rope;  // backward: RoPE table to take dQ and dK back through (null: none)
};

// Query head of workgroup column x of the forward grid: column
// x = m n_kv + j runs head j G + m (G = n_q / n_kv), so the G query heads of
// kv head j are the columns congruent to j modulo n_kv. Workgroups go to the
// eight XCDs in turn by dispatch index; with n_q a multiple of 8 a column's
// XCD is x % 8, and with n_kv dividing 8 every workgroup on XCD c then reads
// kv head c % n_kv: they stream the same K and V tiles and share them in L2.
// (The dQ kernel, whose streamed tiles are the same, measured no gain from
// it and keeps column = head.)
__device__ __forceinline__ int head_of_column(int x, int nq, int nkv) {
  const int g = nq / nkv;
  return (x % nkv) * g + x / nkv;
}

// ---------------------------------------------------------------------------
// backward preprocessing: Dr[h][t] = sum_d dO[t, h, d] * O[t, h, d]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void flash_bwd_dot_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                           float* __restrict__ Dr, int T, int nq) {
  // 16 threads per (token, head) row of 128 elements
  const int64_t row = (int64_t)blockIdx.x * (NT / 16) + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  float s = 0.f;
  if (row < (int64_t)T * nq) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(o + row * D + 8 * c);
    const u32x4_t g = *reinterpret_cast<const u32x4_t*>(dout + row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(g[i] << 16), s);
      s = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(g[i] & 0xffff0000u), s);
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 16);
  if (c == 0 && row < (int64_t)T * nq) {
    const int64_t t = row / nq, hh = row % nq;
    Dr[hh * T + t] = s;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 128 keys of one kv head, streaming 64-query tiles of
// every query head of the group; wave w owns 32 keys, whose K and V rows it
// holds in registers and whose dK and dV it accumulates.
//
// The query tiles (Q and dO rows, their lse and D values) go from global
// memory straight into a ring of three LDS stages (buffer loads with the LDS
// as destination, no registers on the way), two tiles ahead of the one being
// computed. Only the row-major image is stored: the transposed operands of
// the dV and dK products are read from it with the transposing LDS read
// (ds_read_b64_tr_b16), so no wave spends vector instructions on transposes.
// A manual barrier (wait for this wave's loads of the next tile, then
// s_barrier) replaces __syncthreads, whose fence would also wait for the
// loads two tiles ahead.
// ---------------------------------------------------------------------------

// row-major [64 rows][128] bf16 stage tile: 256-byte rows of 16 chunks of 16
// bytes, chunk c of row r stored at position c ^ g(r), where g swaps the two
// 2-bit halves of r % 16. It is a bijection of r % 16, so 16 consecutive rows
// with one chunk each (a 16-byte fragment read of 16 lanes) hit 16 distinct
// positions; and the four rows 4a .. 4a + 3 get distinct high bits, so those
// rows together with chunks 4m .. 4m + 3 (a transposing 8-byte read of 32
// lanes) hit 16 distinct positions too.
__device__ __forceinline__ int dr_swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }
__device__ __forceinline__ int dr_off(int row, int c16) { return row * 256 + ((c16 ^ dr_swz(row)) << 4); }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t* lds_bf16x4_t;

// s_waitcnt: at most n vector-memory operations outstanding and no LDS
// operation (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Buffer resource over `bytes` bytes at base (raw buffer: offsets at or past
// `bytes` read as zeros).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xffff, (int)bytes, 0x00020000};
}
// One 16-byte-per-lane load from global memory straight into LDS: lane L's
// 16 bytes (at voff of the buffer) land at lds + 16 L. Written as inline
// assembly on purpose: for the builtin form the compiler makes every later
// LDS read it cannot tell apart from the destination wait for all loads in
// flight, which would drain the loads issued two tiles ahead. The kernels
// therefore count these loads themselves (s_waitcnt before each barrier) and
// wait for all their own register loads before issuing the first one, so no
// wait the compiler places for a register load can fall inside the loop.
__device__ __forceinline__ void dma16(i32x4_t r, const void* lds, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  // An SALU write of M0 needs one wait state before a load that writes LDS.
  // M0 cannot be declared clobbered (the compiler reserves it and ignores
  // the clobber); the kernels that call this use M0 nowhere else (their
  // code has no other M0 access), and each call sets it afresh.
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}

// A operand of a dV / dK product from a row-major stage tile: d-row
// 32 dt + (lane % 32), k-step j of 32-row sub-tile u (rows 32u + 16j +
// {4h .. 4h + 3, 8 + 4h .. 8 + 4h + 3}), as two transposing reads. In a read,
// lane c of each 16-lane group addresses 4 consecutive d of one row and
// receives, in slot k, element c % 4 of the chunk addressed by lane
// 4k + c / 4: so lane c of the group addresses row r0 + c / 4, d
// d0 + 4 (c % 4), and every lane receives its own d for rows r0 .. r0 + 3.
// The swizzle term of such a row depends on the lane only (r % 4 = (c / 4)
// % 4 and (r / 4) % 4 = h, or h + 2 for the rows 8 further), and the d-tile
// dt enters the chunk index as 4 dt, which XORs into it bit for bit; so the
// lane's offsets for the four d-tiles are computed once (TrBase) and a read
// adds only the sub-tile's and k-step's row offset, an immediate.
struct TrBase {
  int b0[4], b1[4];  // rows r and r + 8 of sub-tile 0, k-step 0, for d-tile dt
};
__device__ __forceinline__ TrBase tr_base(int lane) {
  const int grp = lane >> 4, c = lane & 15, h = lane >> 5;
  const int s0 = 4 * ((c >> 2) & 3) + h;           // dr_swz of row r; row r + 8: s0 ^ 2
  const int x = 2 * (grp & 1) + ((c & 3) >> 1);    // chunk of d within the d-tile
  const int l = (4 * h + (c >> 2)) * 256 + (c & 1) * 8;
  TrBase b;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    b.b0[dt] = l + (((4 * dt) ^ x ^ s0) << 4);
    b.b1[dt] = l + 8 * 256 + (((4 * dt) ^ x ^ s0 ^ 2) << 4);
  }
  return b;
}
__device__ __forceinline__ bf16x8_t rd_trl(const char* t, const TrBase& tb, int dt, int u, int j) {
  const char* row = t + (32 * u + 16 * j) * 256;
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(row + tb.b0[dt]));
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(row + tb.b1[dt]));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand of a score product: rows 32u + (lane % 32), d-step s
__device__ __forceinline__ bf16x8_t rd_rml(const char* t, int u, int s, int lane) {
  const int row = 32 * u + (lane & 31);
  return *reinterpret_cast<const bf16x8_t*>(t + dr_off(row, 2 * s + (lane >> 5)));
}

__global__ __launch_bounds__(NT) void flash_dkdv_kernel(FlashParams p, const bf16* __restrict__ dout,
                                                        const float* __restrict__ lse, const float* __restrict__ Dr,
                                                        bf16* __restrict__ dqkv) {
  constexpr int NST = 3;                                   // LDS stages
  constexpr int STAGE = 2 * TILE * 256;                    // Q, dO
  constexpr int NDMA = 10;                                 // loads per wave per tile (8 rows, 2 statistics)
  extern __shared__ __align__(16) char smem[];
  __shared__ __align__(16) float sstat[NST][2 * TILE];   // lse and D of each stage's queries
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(tid), h = lane >> 5, n = lane & 31;
  const TrBase tb = tr_base(lane);
  const int hk = blockIdx.x, b = blockIdx.z;
  const int kb = blockIdx.y;  // earliest keys (most queries) first
  const int G = p.nq / p.nkv;
  const int T = gridDim.z * p.seq;
  const bf16* base = p.qkv + (int64_t)b * p.seq * p.ld;
  const int64_t ldo = (int64_t)p.nq * D;
  const bf16* dob = dout + (int64_t)b * p.seq * ldo;
  const int k0 = kb * BROWS, kw = k0 + w * WROWS, kpos = kw + n;
  const int kcol = (p.nq + hk) * D, vcol = (p.nq + p.nkv + hk) * D;

  bf16x8_t kf[8], vf[8];
  load_rows_b(kf, base, p.ld, kpos, p.seq, kcol, h);
  load_rows_b(vf, base, p.ld, kpos, p.seq, vcol, h);
  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dk[i] = dv[i] = zero16();
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // K and V landed (see dma16)

  // the streamed tiles: query tile qt of head g covers queries [k0 + 64 qt, +64)
  const int nqt = (p.seq - k0 + TILE - 1) / TILE;
  const int ntile = G * nqt;
  // Tile i (clamped to the last one: the loads past the end repeat it into a
  // stage nobody reads, which keeps every wave's count of loads uniform) goes
  // into stage i % NST. Wave w loads rows 16w .. 16w + 15 of Q and dO (four
  // 1 KB instructions each: lane L writes 16 bytes at row 4j + L / 16,
  // position L % 16, so it loads chunk (L % 16) ^ g(row)). Rows at or past
  // the sequence end read as zeros (each tile's buffer resources end at its
  // last valid row). The lse and D rows 16w .. 16w + 15 go through registers
  // of lanes 0..15, loaded one tile before they are stored.
  auto tile_rows = [&](int i, int& q0, int& head, int& nvalid) __attribute__((always_inline)) {
    const int ic = min(i, ntile - 1);
    const int g = ic / nqt;
    q0 = k0 + (ic % nqt) * TILE;
    head = hk * G + g;
    nvalid = min(TILE, p.seq - q0);
  };
  auto issue = [&](int i) __attribute__((always_inline)) {
    int q0, head, nvalid;
    tile_rows(i, q0, head, nvalid);
    char* st = smem + (i % NST) * STAGE;
    const i32x4_t rq = rsrc4(base + (int64_t)q0 * p.ld + head * D, (uint32_t)((nvalid - 1) * p.ld * 2 + 256));
    const i32x4_t ro = rsrc4(dob + (int64_t)q0 * ldo + head * D, (uint32_t)((nvalid - 1) * ldo * 2 + 256));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * w + 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ dr_swz(row);
      // a row past the end gets an offset past every buffer's range: zeros
      const uint32_t oq = row < nvalid ? (uint32_t)(row * p.ld * 2 + c * 16) : 0x80000000u;
      const uint32_t oo = row < nvalid ? (uint32_t)(row * ldo * 2 + c * 16) : 0x80000000u;
      dma16(rq, st + (16 * w + 4 * j) * 256, oq);
      dma16(ro, st + TILE * 256 + (16 * w + 4 * j) * 256, oo);
    }
  };
  float ls = 0.f, dsv = 0.f;  // lanes 0..15: lse and D of row 16w + lane of the tile being staged
  auto fetch_stats = [&](int i) __attribute__((always_inline)) {
    int q0, head, nvalid;
    tile_rows(i, q0, head, nvalid);
    if (lane < 16) {
      const int r = min(16 * w + lane, nvalid - 1);  // rows past the end: any finite value (masked)
      const int64_t si = (int64_t)head * T + (int64_t)b * p.seq + q0 + r;
      ls = lse[si];
      dsv = Dr[si];
    }
  };
  auto put_stats = [&](int i) __attribute__((always_inline)) {
    float* sl = sstat[i % NST];
    if (lane < 16) {
      sl[16 * w + lane] = ls;
      sl[TILE + 16 * w + lane] = dsv;
    }
  };
  // this wave's loads of the next tile landed (the NDMA loads issued since
  // may still be in flight), its LDS operations done, then all waves
  auto sync_next = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NDMA));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  fetch_stats(0);
  put_stats(0);
  fetch_stats(1);
  put_stats(1);
  issue(0);
  issue(1);
  fetch_stats(2);
  sync_next();

  // lse (in log2 units) and D of the 16 queries of sub-tile u that a lane's
  // score registers hold: registers 4g .. 4g + 3 are queries
  // 32u + 8g + 4h + 0..3, one 16-byte read each
  auto stats = [&](float4 (&lq)[4], float4 (&dq)[4], int u, const float* sL) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 l = *reinterpret_cast<const float4*>(sL + 32 * u + 8 * g + 4 * h);
      lq[g] = make_float4(l.x * LOG2E, l.y * LOG2E, l.z * LOG2E, l.w * LOG2E);
      dq[g] = *reinterpret_cast<const float4*>(sL + TILE + 32 * u + 8 * g + 4 * h);
    }
  };
  // probabilities P and dS = P (dP - D) of sub-tile u of the query tile at
  // q0 from its scores st and dp, packed as the bf16 operands of the dV and
  // dK products (k-steps j = 0, 1)
  auto probs = [&](const f32x16_t& st, const f32x16_t& dp, bf16x8_t (&pb)[2], bf16x8_t (&sb)[2],
                   const float4 (&lq)[4], const float4 (&dq)[4], int u, int q0, auto mask_c)
                   __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float pr[8], ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * j + i;
        pr[i] = fexp2(st[r] * p.c2 - lane_of(lq[r >> 2], r & 3));
        if constexpr (MASK) {  // kpos > q only on the diagonal
          const int q = q0 + 32 * u + 8 * (r >> 2) + 4 * h + (r & 3);
          if (kpos > q || q >= p.seq) pr[i] = 0.f;
        }
        ds[i] = pr[i] * (dp[r] - lane_of(dq[r >> 2], r & 3));
      }
      u32x4_t a, c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
        c[i] = pack_bf16x2(ds[2 * i], ds[2 * i + 1]);
      }
      pb[j] = __builtin_bit_cast(bf16x8_t, a);
      sb[j] = __builtin_bit_cast(bf16x8_t, c);
    }
  };

  // one query tile; MASK: the tile holds queries before some key of the
  // wave (the diagonal) or past the sequence end. Separate loops per variant
  // keep the masking code out of the interior tiles.
  auto tile = [&](int it, auto mask_c) __attribute__((always_inline)) {
    const int q0 = k0 + (it % nqt) * TILE;
    const char* sQ = smem + (it % NST) * STAGE;
    const char* sO = sQ + TILE * 256;
    const float* sL = sstat[it % NST];
    if (!decltype(mask_c)::value || q0 + TILE - 1 >= kw) {  // else every query of the tile is before every key of the wave
      // The two 32-query sub-tiles u = 0, 1, each in three phases: P(u) the
      // score products S = Q K^T and dP = dO V^T (16 MFMAs), E(u) the
      // probabilities and dS on the vector ALU, D(u) the dV and dK products
      // (16 MFMAs). With one wave per SIMD the vector work hides only under
      // MFMAs of the same wave, so the phases run as P(0); P(1) with E(0);
      // D(0) with E(1); D(1); LDS reads are issued a phase ahead.
      bf16x8_t fq[8], fo[8], tq[2][4], to[2][4];
      f32x16_t st0 = zero16(), dp0 = zero16(), st1 = zero16(), dp1 = zero16();
      bf16x8_t pb0[2], sb0[2], pb1[2], sb1[2];
      float4 lq0[4], dq0[4], lq1[4], dq1[4];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        fq[s] = rd_rml(sQ, 0, s, lane);
        fo[s] = rd_rml(sO, 0, s, lane);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        st0 = mfma(fq[s], kf[s], st0);
        dp0 = mfma(fo[s], vf[s], dp0);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        fq[s] = rd_rml(sQ, 1, s, lane);
        fo[s] = rd_rml(sO, 1, s, lane);
      }
      stats(lq0, dq0, 0, sL);
      __builtin_amdgcn_sched_barrier(0);
      // P(1) with E(0); sub-tile 0's transposed operands load meanwhile
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        st1 = mfma(fq[s], kf[s], st1);
        dp1 = mfma(fo[s], vf[s], dp1);
      }
      probs(st0, dp0, pb0, sb0, lq0, dq0, 0, q0, mask_c);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          to[j][dt] = rd_trl(sO, tb, dt, 0, j);
          tq[j][dt] = rd_trl(sQ, tb, dt, 0, j);
        }
      stats(lq1, dq1, 1, sL);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA,
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // up to eight vector ops,
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
      }
      __builtin_amdgcn_sched_barrier(0);
      // D(0) with E(1); sub-tile 1's transposed operands load meanwhile
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          dv[dt] = mfma(to[j][dt], pb0[j], dv[dt]);
          dk[dt] = mfma(tq[j][dt], sb0[j], dk[dt]);
        }
      probs(st1, dp1, pb1, sb1, lq1, dq1, 1, q0, mask_c);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          to[j][dt] = rd_trl(sO, tb, dt, 1, j);
          tq[j][dt] = rd_trl(sQ, tb, dt, 1, j);
        }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // D(1), then the loads of the tile two ahead
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          dv[dt] = mfma(to[j][dt], pb1[j], dv[dt]);
          dk[dt] = mfma(tq[j][dt], sb1[j], dk[dt]);
        }
    }
    // tile it + 2 into the stage of tile it - 1, which every wave left before
    // the last barrier: its statistics (loaded a tile ago), its rows, then
    // the statistics of the tile after it
    put_stats(it + 2);
    issue(it + 2);
    fetch_stats(it + 3);
    sync_next();
  };
  // per query head: tiles qt < qa reach the wave's diagonal (q0 < kw + WROWS
  // - 1), tiles qt >= qb pass the sequence end (q0 + TILE > seq)
  const int qa = min(nqt, (kw + WROWS - 1 - k0 + TILE - 1) / TILE);
  const int qb = max(qa, (p.seq - k0) / TILE);
  for (int g = 0; g < G; ++g) {
    int qt = 0;
    for (; qt < qa; ++qt) tile(g * nqt + qt, std::true_type{});
    for (; qt < qb; ++qt) tile(g * nqt + qt, std::false_type{});
    for (; qt < nqt; ++qt) tile(g * nqt + qt, std::true_type{});
  }
  // drain the loads past the end before the workgroup exits
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  bf16* dst = dqkv + (int64_t)b * p.seq * p.ld;
  store_acc_rows(dk, p.scale, dst, p.ld, kpos, p.seq, kcol, h, p.rope);
  store_acc_rows(dv, 1.f, dst, p.ld, kpos, p.seq, vcol, h);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup = 128 queries of one head, streaming 64-key tiles of its
// kv head (K and V rows) through the same three-stage LDS ring as the dK/dV
// kernel (direct loads, row-major image only, K^T operands by transposing
// reads); wave w owns 32 queries, whose Q and dO rows it holds in registers
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void flash_dq_kernel(FlashParams p, const bf16* __restrict__ dout,
                                                      const float* __restrict__ lse, const float* __restrict__ Dr,
                                                      bf16* __restrict__ dqkv) {
  constexpr int NST = 3;
  constexpr int STAGE = 2 * TILE * 256;  // K, V
  constexpr int NDMA = 8;                // loads per wave per tile
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(tid), h = lane >> 5, n = lane & 31;
  const TrBase tb = tr_base(lane);
  const int head = blockIdx.x, b = blockIdx.z;
  const int qb = p.n_blocks - 1 - blockIdx.y;  // longest rows first
  const int hk = head / (p.nq / p.nkv);
  const int T = gridDim.z * p.seq;
  const bf16* base = p.qkv + (int64_t)b * p.seq * p.ld;
  const int q0 = qb * BROWS, qw = q0 + w * WROWS, qpos = qw + n;
  const int kcol = (p.nq + hk) * D, vcol = (p.nq + p.nkv + hk) * D;
  const int64_t ldo = (int64_t)p.nq * D;

  bf16x8_t qf[8], dof[8];
  load_rows_b(qf, base, p.ld, qpos, p.seq, head * D, h);
  load_rows_b(dof, dout + (int64_t)b * p.seq * ldo, ldo, qpos, p.seq, head * D, h);
  const int64_t si = (int64_t)head * T + (int64_t)b * p.seq + min(qpos, p.seq - 1);
  const float l2 = lse[si] * LOG2E, dd = Dr[si];
  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // Q, dO, lse and D landed (see dma16)
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    to_acc_regs(qf[s]);
    to_acc_regs(dof[s]);
  }

  const int klast = min(q0 + BROWS, p.seq) - 1;
  const int ntile = klast / TILE + 1;
  // key tile i (clamped as in the dK/dV kernel) into stage i % NST: wave w
  // loads rows 16w .. 16w + 15 of K and V
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int k0 = min(i, ntile - 1) * TILE;
    const int nvalid = min(TILE, p.seq - k0);
    char* st = smem + (i % NST) * STAGE;
    const i32x4_t rk = rsrc4(base + (int64_t)k0 * p.ld + kcol, (uint32_t)((nvalid - 1) * p.ld * 2 + 256));
    const i32x4_t rv = rsrc4(base + (int64_t)k0 * p.ld + vcol, (uint32_t)((nvalid - 1) * p.ld * 2 + 256));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * w + 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ dr_swz(row);
      const uint32_t off = row < nvalid ? (uint32_t)(row * p.ld * 2 + c * 16) : 0x80000000u;
      dma16(rk, st + (16 * w + 4 * j) * 256, off);
      dma16(rv, st + TILE * 256 + (16 * w + 4 * j) * 256, off);
    }
  };
  auto sync_next = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NDMA));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  issue(0);
  issue(1);
  sync_next();

  // dS of 32-key sub-tile t of the key tile at k0 from its scores, packed as
  // the bf16 B operands of the dQ product (k-steps j = 0, 1)
  auto dscore = [&](const f32x16_t& st, const f32x16_t& dp, bf16x8_t (&sb)[2], int t, int k0, auto mask_c)
                    __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float ds[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * j + i;
        float pr = fexp2(st[r] * p.c2 - l2);
        if constexpr (MASK) {
          const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > qpos) pr = 0.f;
        }
        ds[i] = pr * (dp[r] - dd);
      }
      u32x4_t c;
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = pack_bf16x2(ds[2 * i], ds[2 * i + 1]);
      sb[j] = __builtin_bit_cast(bf16x8_t, c);
    }
  };
  // one key tile; MASK as in the forward (separate loops, see there). The two
  // 32-key sub-tiles run as P(0); P(1) with E(0); D(0) with E(1); D(1), where
  // P is the score products S = K Q^T and dP = V dO^T (16 MFMAs), E the dS
  // arithmetic and D the dQ product (8 MFMAs).
  auto tile = [&](int kt, auto mask_c) __attribute__((always_inline)) {
    const int k0 = kt * TILE;
    const char* sK = smem + (kt % NST) * STAGE;
    const char* sV = sK + TILE * 256;
    if (!decltype(mask_c)::value || k0 <= qw + WROWS - 1) {
      bf16x8_t fk[8], fv[8], tk[2][4];
      f32x16_t st0 = zero16(), dp0 = zero16(), st1 = zero16(), dp1 = zero16();
      bf16x8_t sb0[2], sb1[2];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        fk[s] = rd_rml(sK, 0, s, lane);
        fv[s] = rd_rml(sV, 0, s, lane);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        st0 = mfma(fk[s], qf[s], st0);
        dp0 = mfma(fv[s], dof[s], dp0);
      }
      to_arch_regs(st0);
      to_arch_regs(dp0);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        fk[s] = rd_rml(sK, 1, s, lane);
        fv[s] = rd_rml(sV, 1, s, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        st1 = mfma(fk[s], qf[s], st1);
        dp1 = mfma(fv[s], dof[s], dp1);
      }
      to_arch_regs(st1);
      to_arch_regs(dp1);
      dscore(st0, dp0, sb0, 0, k0, mask_c);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) tk[j][dt] = rd_trl(sK, tb, dt, 0, j);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA,
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // up to three vector ops,
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // an LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(tk[j][dt], sb0[j], acc[dt]);
      dscore(st1, dp1, sb1, 1, k0, mask_c);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) tk[j][dt] = rd_trl(sK, tb, dt, 1, j);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(tk[j][dt], sb1[j], acc[dt]);
    }
    issue(kt + 2);
    sync_next();
  };
  const int kfree = min(ntile, (qw + 1) / TILE);
  int kt = 0;
  for (; kt < kfree; ++kt) tile(kt, std::false_type{});
  for (; kt < ntile; ++kt) tile(kt, std::true_type{});
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  store_acc_rows(acc, p.scale, dqkv + (int64_t)b * p.seq * p.ld, p.ld, qpos, p.seq, head * D, h, p.rope);
}

// ---------------------------------------------------------------------------
// forward: one workgroup = 128 queries of one head; wave w owns 32 of them.
// The key tiles (K and V rows) go from global memory straight into two LDS
// stages (the backward kernels' direct loads and row-major layout; V^T
// operands by transposing reads): tile kt + 1 is loaded while tile kt is
// computed, one barrier per tile. Registers are capped for two waves per
// SIMD, so two workgroups share a CU and one's softmax overlaps the other's
// MFMAs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_fwd_kernel(
    FlashParams p, bf16* __restrict__ o, float* __restrict__ lse) {
  constexpr int STAGE = 2 * TILE * 256;  // K, V
  __shared__ __align__(16) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(tid), h = lane >> 5, n = lane & 31;
  const TrBase tb = tr_base(lane);
  const int head = head_of_column(blockIdx.x, p.nq, p.nkv), b = blockIdx.z;
  const int qb = p.n_blocks - 1 - blockIdx.y;  // longest rows first
  const int hk = head / (p.nq / p.nkv);
  const bf16* base = p.qkv + (int64_t)b * p.seq * p.ld;
  const int q0 = qb * BROWS, qw = q0 + w * WROWS, qpos = qw + n;
  const int kcol = (p.nq + hk) * D, vcol = (p.nq + p.nkv + hk) * D;

  bf16x8_t qf[8];
  load_rows_b(qf, base, p.ld, qpos, p.seq, head * D, h);
  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  float m = -INFINITY, l = 0.f;
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // Q landed (see dma16)

  const int klast = min(q0 + BROWS, p.seq) - 1;
  const int ntile = klast / TILE + 1;
  // key tile i (clamped to the last one) into stage i & 1: wave w loads
  // rows 16w .. 16w + 15 of K and V
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int k0 = min(i, ntile - 1) * TILE;
    const int nvalid = min(TILE, p.seq - k0);
    char* st = smem + (i & 1) * STAGE;
    const i32x4_t rk = rsrc4(base + (int64_t)k0 * p.ld + kcol, (uint32_t)((nvalid - 1) * p.ld * 2 + 256));
    const i32x4_t rv = rsrc4(base + (int64_t)k0 * p.ld + vcol, (uint32_t)((nvalid - 1) * p.ld * 2 + 256));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * w + 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ dr_swz(row);
      const uint32_t off = row < nvalid ? (uint32_t)(row * p.ld * 2 + c * 16) : 0x80000000u;
      dma16(rk, st + (16 * w + 4 * j) * 256, off);
      dma16(rv, st + TILE * 256 + (16 * w + 4 * j) * 256, off);
    }
  };
  // this wave's loads of the next tile landed, its LDS reads done, then all
  auto sync_next = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  issue(0);
  sync_next();
  // one key tile; MASK: the tile reaches past the wave's first query (the
  // last one or two tiles; keys past the sequence end fall in them too, since
  // every query is before the end). The two variants are separate loops so
  // that the interior tiles carry no masking code at all.
  auto tile = [&](int kt, auto mask_c) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int k0 = kt * TILE;
    const char* sK = smem + (kt & 1) * STAGE;
    const char* sV = sK + TILE * 256;
    issue(kt + 1);  // into the other stage, which every wave left before the last barrier
    if (!MASK || k0 <= qw + WROWS - 1) {  // else every key of the tile is after every query of the wave
      f32x16_t st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[t] = zero16();
#pragma unroll
        for (int s = 0; s < 8; ++s) st[t] = mfma(rd_rml(sK, t, s, lane), qf[s], st[t]);
      }
      float mx = -INFINITY;
      if constexpr (MASK) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
            const float v = key > qpos ? -INFINITY : st[t][r] * p.c2;
            st[t][r] = v;
            mx = fmaxf(mx, v);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            st[t][r] *= p.c2;
            mx = fmaxf(mx, st[t][r]);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // The running max moves only when some lane's tile max exceeds it by
      // more than 2^RESCALE_LOG2: until then the probabilities are taken
      // against the stale max (each at most 2^RESCALE_LOG2, exact in fp32 and
      // as bf16 operands), which leaves l, acc and lse = m + log2(l)
      // unchanged and skips the rescale of the accumulator on most tiles.
      // Tile 0 holds key 0 <= every query, so m is finite after it.
      if (__builtin_amdgcn_ballot_w64(mx > m + RESCALE_LOG2) != 0) {  // uniform over the wave
        const float mn = fmaxf(m, mx);
        const float alpha = fexp2(m - mn);
        l *= alpha;
        m = mn;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      }
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fexp2(st[t][r] - m);
          st[t][r] = e;
          sum += e;
        }
      sum += __shfl_xor(sum, 32, 64);
      l += sum;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_t pb = to_operand(st[t], j);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(rd_trl(sV, tb, dt, t, j), pb, acc[dt]);
        }
    }
    sync_next();
  };
  // tiles wholly at or before the wave's first query: k0 + TILE - 1 <= qw
  const int kfree = min(ntile, (qw + 1) / TILE);
  int kt = 0;
  for (; kt < kfree; ++kt) tile(kt, std::false_type{});
  for (; kt < ntile; ++kt) tile(kt, std::true_type{});
  const float inv = 1.f / l;
  store_acc_rows(acc, inv, o + (int64_t)b * p.seq * p.nq * D, (int64_t)p.nq * D, qpos, p.seq, head * D, h);
  if (h == 0 && qpos < p.seq) lse[(int64_t)head * gridDim.z * p.seq + (int64_t)b * p.seq + qpos] = (m + __log2f(l)) * LN2;
}

FlashParams make_params(const AttnDesc& a, const void* qkv) {
  FlashParams p;
  p.qkv = reinterpret_cast<const bf16*>(qkv);
  p.ld = (int64_t)(a.n_q + 2 * a.n_kv) * D;
  p.seq = a.seq;
  p.nq = a.n_q;
  p.nkv = a.n_kv;
  p.scale = 1.0f / sqrtf((float)D);
  p.c2 = p.scale * LOG2E;
  p.n_blocks = (int)cdiv(a.seq, BROWS);
  p.rope = nullptr;
  return p;
}

double causal_pairs(const AttnDesc& a) { return (double)a.batch * a.seq * (a.seq + 1.0) / 2.0; }

// double-buffered LDS stages of the backward kernels (above the 64 KB static limit)
constexpr size_t DQ_LDS = 3 * 2 * TILE * 256;
constexpr size_t DKDV_LDS = 3 * 2 * TILE * 256;  // plus the kernel's static statistics array

rp_status set_lds_limits() {
  static bool done = false;
  if (!done) {
    RP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&flash_dq_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)DQ_LDS));
    RP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&flash_dkdv_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)DKDV_LDS));
    done = true;
  }
  return RP_OK;
}

}  // namespace

bool flash_supported(const AttnDesc& a) {
  return a.dt == RP_DTYPE_BF16 && a.d == D && a.n_kv > 0 && a.n_q % a.n_kv == 0 && a.seq >= 1;
}

rp_status flash_fwd(const AttnDesc& a, const void* qkv, void* o, float* lse, hipStream_t s) {
  RP_CHECK(((uintptr_t)qkv & 15) == 0 && ((uintptr_t)o & 15) == 0, RP_ERR_INVALID,
           "flash attention: qkv and o must be 16-byte aligned");
  const FlashParams p = make_params(a, qkv);
  TraceScope ts(s, "flash_fwd_kernel", 4.0 * D * a.n_q * causal_pairs(a), 0.0);
  RP_LAUNCH(flash_fwd_kernel, dim3(a.n_q, p.n_blocks, a.batch), dim3(NT), 0, s, p, (bf16*)o, lse);
  return RP_OK;
}

rp_status flash_bwd(const AttnDesc& a, const void* qkv, const void* o, const void* dout, const float* lse,
                    float* Dbuf, void* dqkv, hipStream_t s, const float2* rope_inv) {
  RP_CHECK(((uintptr_t)qkv & 15) == 0 && ((uintptr_t)o & 15) == 0 && ((uintptr_t)dout & 15) == 0 &&
               ((uintptr_t)dqkv & 15) == 0,
           RP_ERR_INVALID, "flash attention: buffers must be 16-byte aligned");
  RP_CHECK(((uintptr_t)rope_inv & 15) == 0, RP_ERR_INVALID, "flash attention: the RoPE table must be 16-byte aligned");
  RP_TRY(set_lds_limits());
  FlashParams p = make_params(a, qkv);
  p.rope = rope_inv;
  const int T = a.batch * a.seq;
  const int64_t rows = (int64_t)T * a.n_q;
  {
    TraceScope ts(s, "flash_bwd_dot_kernel", 0.0, (double)rows * (2 * D * 2 + 4));
    RP_LAUNCH(flash_bwd_dot_kernel, dim3((unsigned)cdiv(rows, NT / 16)), dim3(NT), 0, s, (const bf16*)o,
              (const bf16*)dout, Dbuf, T, a.n_q);
  }
  {
    // dV = P^T dO and dK = dS^T Q: two of the four backward products
    TraceScope ts(s, "flash_dkdv_kernel", 4.0 * D * a.n_q * causal_pairs(a), 0.0);
    RP_LAUNCH(flash_dkdv_kernel, dim3(a.n_kv, p.n_blocks, a.batch), dim3(NT), DKDV_LDS, s, p, (const bf16*)dout, lse,
              Dbuf, (bf16*)dqkv);
  }
  {
    // dQ = dS K and dP = dO V^T: the other two
    TraceScope ts(s, "flash_dq_kernel", 4.0 * D * a.n_q * causal_pairs(a), 0.0);
    RP_LAUNCH(flash_dq_kernel, dim3(a.n_q, p.n_blocks, a.batch), dim3(NT), DQ_LDS, s, p, (const bf16*)dout, lse, Dbuf,
              (bf16*)dqkv);
  }
  return RP_OK;
}

}  // namespace rp
