// GEMMs of the stage: every projection of the decoder layer (q/k/v, o, gate/up,
// down), their input-gradient (NN) and weight-gradient (TN) products, and the
// LM-head shard products. These are the dense contractions that carry almost
// all of a layer's FLOPs (the paper's appendix C counts matrix multiplies only).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on gfx950. WGM x WGN waves per
// workgroup (2 x 4 for the 256 x 256 tiles of the large products), each
// owning a (BM/WGM) x (BN/WGN) block of 32x32 MFMA tiles.
// K advances 64 at a time through double-buffered LDS (one barrier per step):
// the next step's global loads are issued before the current step's MFMAs.
// Both kinds of operand are copied 16 bytes at a time and stored into LDS as
// they lie in memory: operands whose K is the contiguous dimension as rows of
// 64 k (padded to 144 bytes), operands whose M/N is contiguous (the
// transposed operands of the backward products) as 64 k rows of the tile's
// M/N extent, whose fragments come from gfx950's transposing LDS read. The
// MFMA loop is the same for every layout, and the kernel transposes nothing,
// in registers or otherwise.
// Epilogues fuse the residual add, the SwiGLU activation (gate and up columns
// of one output column are held by the same lane) and its backward, and fp32
// accumulation.
//
// fp32 path (and a bf16 cross-check): a plain LDS-tiled FMA kernel with the
// same epilogue semantics.
#include <type_traits>

#include "ops.h"
#include "trace.h"

namespace rp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BK = 64;

struct GemmParams {
  int M, N, K;
  const bf16* A; int64_t lda;
  const bf16* B; int64_t ldb;
  void* C; int64_t ldc;
  const void* R; int64_t ldr;
  void* C2; int64_t ldc2;
  uint32_t a_bytes, b_bytes;  // extent of A and B (loads beyond read as zero)
  int F;            // SwiGLU width (EPI_SWIGLU: N == 2F; EPI_SWIGLU_BWD: N == F)
  int tiles_m, tiles_n;
  int accumulate;
  float alpha;      // C = alpha * A B^T (+ R) for the store and residual epilogues
  int kc;           // k extent of one split (blockIdx.y); K when not split
  int64_t c_split;  // element stride between the splits' partial outputs
  // grouped mode (one product per expert over its rows; see GemmGroup)
  const int* g_tile_e;    // [tiles_m] expert of each 128/256-row tile, -1 = idle
  const int* g_tile_m0;   // [tiles_m] first row of the tile within its expert
  const int* g_off;       // [E] first row of each expert
  const int* g_cnt;       // [E] rows of each expert
  const int* g_rows;      // gathered A: operand row of each grouped row
  const float* row_scale; // [rows] per-row factor of the epilogue (or null)
  int64_t b_stride;       // elements between consecutive experts' B
  const float2* rope_tab; // EPI_ROPE: (cos, sin) of position p, pair i at [p * 64 + i]
  int rope_seq, rope_heads;
  int vec;  // row strides of C, R and C2 (and F) multiples of 4 elements, bases aligned to 4 elements
  int skip_c;  // EPI_SWIGLU: store only C2
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }

// Four consecutive elements of one row, as fp32 values: one 16-byte (fp32)
// or 8-byte (bf16) access when `vec` (the caller guarantees the alignment),
// else `cnt` (<= 4) single-element accesses.
__device__ __forceinline__ void ld4(const float* q, int cnt, bool vec, float (&v)[4]) {
  if (vec && cnt == 4) {
    const float4 t = *reinterpret_cast<const float4*>(q);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < cnt ? q[e] : 0.f;
  }
}
__device__ __forceinline__ void ld4(const bf16* q, int cnt, bool vec, float (&v)[4]) {
  if (vec && cnt == 4) {
    const u32x2_t t = *reinterpret_cast<const u32x2_t*>(q);
    v[0] = __builtin_bit_cast(float, t[0] << 16); v[1] = __builtin_bit_cast(float, t[0] & 0xffff0000u);
    v[2] = __builtin_bit_cast(float, t[1] << 16); v[3] = __builtin_bit_cast(float, t[1] & 0xffff0000u);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < cnt ? to_f(q[e]) : 0.f;
  }
}
__device__ __forceinline__ void st4(float* q, int cnt, bool vec, const float (&v)[4]) {
  if (vec && cnt == 4) {
    *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < cnt) q[e] = v[e];
  }
}
__device__ __forceinline__ void st4(bf16* q, int cnt, bool vec, const float (&v)[4]) {
  if (vec && cnt == 4) {
    const uint32_t w0 = (uint32_t)to_bf16(v[0]).u | ((uint32_t)to_bf16(v[1]).u << 16);
    const uint32_t w1 = (uint32_t)to_bf16(v[2]).u | ((uint32_t)to_bf16(v[3]).u << 16);
    *reinterpret_cast<u32x2_t*>(q) = u32x2_t{w0, w1};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < cnt) q[e] = to_bf16(v[e]);
  }
}

// Buffer resource over `bytes` bytes at p: loads at offsets >= bytes return 0
// (the hardware range check), so tile rows past the matrix edge read as zeros
// without a branch. The whole offset goes in the per-lane voffset (the range
// check covers it); OOB_SHIFT pushes a chunk that must read as zero out of
// range (operand extents stay below 2^31, so the sum cannot wrap).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t OOB_SHIFT = 0x80000000u;
__device__ __forceinline__ u32x4_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// --- LDS layouts ---------------------------------------------------------------
// A tile holds R rows (M or N index) x 64 k of bf16.
// K-major operands: rows padded to 144 bytes (16-byte chunk kc at row*144 +
// 16*kc); the 8 lanes of a read phase hit 8 distinct 16-byte bank groups and
// fragment addresses step by immediates.
// M-major operands are kept as they lie in memory: 64 k rows of R elements,
// each padded by 64 bytes (2R + 64 bytes a row), so consecutive k rows start
// 64 bytes apart in the 256-byte bank cycle. Fragments come from transposing
// LDS reads (read_mm): a 16-lane group reads 32 bytes of each of four
// consecutive k rows, which the padding puts into four distinct 64-byte bank
// ranges, and the other group of the half-wave reads the next 32 bytes of
// the same rows, so the reads are free of bank conflicts; so are the stores
// of whole rows. The offset is linear in m and k, so a fragment's address is
// the lane's own offset plus an immediate.
template <bool KM> struct Lay;
template <> struct Lay<true> {
  template <int R> static constexpr int BYTES = R * 144;  // tile of R operand rows
  __device__ __forceinline__ static int off(int row, int kc) { return row * 144 + kc * 16; }
};
template <> struct Lay<false> {
  template <int R> static constexpr int BYTES = 64 * (2 * R + 64);  // tile of R operand rows
  template <int R>
  __device__ __forceinline__ static int off(int k, int m) {  // element (m, k)
    return k * (2 * R + 64) + 2 * m;
  }
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t* lds_bf16x4_t;

// Fragment of an M-major operand tile of R rows: operand rows rb + (lane %
// 32), k-substep ks (k = 16 ks + 8 (lane / 32) + 0..7, the order of the
// K-major fragments), as two transposing reads (ds_read_b64_tr_b16). In such
// a read, lane c of each 16-lane group addresses 4 consecutive elements of
// one k row and receives, in slot j, element c % 4 of the 4 addressed by lane
// 4j + c / 4; so lane c addresses k row k0 + c / 4 at m0 + 4 (c % 4), and
// every lane receives its own m for k rows k0 .. k0 + 3.
template <int R>
__device__ __forceinline__ bf16x8_t read_mm(const char* t, int rb, int ks, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const int m = rb + 16 * (g & 1) + 4 * (c & 3);
  const int k = 16 * ks + 8 * (lane >> 5) + (c >> 2);
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(t + Lay<false>::off<R>(k, m)));
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(t + Lay<false>::off<R>(k + 4, m)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// --- global -> register -> LDS copies --------------------------------------

// K-major operand: element (r, k) at g[r * ld + k]; R rows per tile, NT
// threads. SWIGLU: tile row r of wave column w = r / wn_span holds gate row f
// (first half of the span) or up row F + f (second half), so one lane ends up
// with the gate and up pre-activations of the same output column.
// Row maps of a K-major operand tile
enum RowMode {
  ROWS_CONTIG = 0,  // tile row r is operand row row0 + r
  ROWS_SWIGLU = 1,  // gate/up interleave (see LoaderK)
  ROWS_GATHER = 2,  // tile row r is operand row rows[row0 + r] (rows past nrows read as zeros)
  ROWS_ROPE = 3     // rotation pairs: see LoaderK
};

// K-major operand: element (r, k) at g[r * ld + k]; R rows per tile, NT
// threads. ROWS_SWIGLU: tile row r of wave column w = r / wn_span holds gate
// row f (first half of the span) or up row F + f (second half), so one lane
// ends up with the gate and up pre-activations of the same output column.
// ROWS_ROPE (64-row wave spans, heads of 128 rows): wave column w covers dims
// 32 (w % 2) + [0, 32) of head w / 2 of the tile in the first half of its
// span and the same dims + 64 in the second, so one lane holds both members
// of every rotation pair; rows at or past F (the product's N) read as zeros.
template <int R, int MODE, int NT>
struct LoaderK {
  static_assert(R * 8 % NT == 0, "tile rows x 8 chunks must split evenly over the threads");
  static constexpr int NCH = R * 8 / NT;
  static constexpr bool MAPPED = MODE != ROWS_CONTIG;
  u32x4_t reg[NCH];
  uint32_t voff[MAPPED ? NCH : 1];
  uint32_t rstride;    // bytes between this thread's consecutive rows
  int kcol;            // first k of this thread's chunk
  __device__ __forceinline__ void init(int64_t ld, int row0, int tid, int F, int wn_span, const int* rows = nullptr,
                                       int nrows = 0) {
    kcol = (tid & 7) * 8;
    rstride = (uint32_t)((NT / 8) * ld * 2);
    if constexpr (MODE == ROWS_ROPE) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int r = (tid >> 3) + i * (NT / 8);
        const int w = r / wn_span, j = r % wn_span;
        const int grow = row0 + (w >> 1) * 128 + (w & 1) * 32 + (j & 31) + (j >> 5) * 64;
        voff[i] = grow < F ? (uint32_t)(((int64_t)grow * ld + (tid & 7) * 8) * 2) : OOB_SHIFT;
      }
    } else if constexpr (MODE == ROWS_SWIGLU) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int r = (tid >> 3) + i * (NT / 8);
        const int w = r / wn_span, j = r % wn_span, half = wn_span >> 1;
        const int f = row0 + w * half + (j < half ? j : j - half);
        // rows f >= F read garbage of valid rows (or zeros): they only feed
        // output columns >= F, which are never stored
        const int grow = (j < half) ? f : F + f;
        voff[i] = (uint32_t)(((int64_t)grow * ld + (tid & 7) * 8) * 2);
      }
    } else if constexpr (MODE == ROWS_GATHER) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int r = row0 + (tid >> 3) + i * (NT / 8);
        voff[i] = r < nrows ? (uint32_t)(((int64_t)rows[r] * ld + (tid & 7) * 8) * 2) : OOB_SHIFT;
      }
    } else {
      voff[0] = (uint32_t)(((int64_t)(row0 + (tid >> 3)) * ld + (tid & 7) * 8) * 2);
    }
  }
  // issue units: unit u is one 16-byte chunk (load) / one LDS store
  static constexpr int NUNIT = NCH;
  __device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int K, int i) {
    // a chunk past K (the K tail) reads as zeros
    const uint32_t base = (uint32_t)(k0 * 2) + (k0 + kcol < K ? 0u : OOB_SHIFT);
    reg[i] = bload(rs, base + (MAPPED ? voff[i] : voff[0] + (uint32_t)i * rstride));
  }
  __device__ __forceinline__ void store_unit(char* lds, int tid, int i) {
    const int r = (tid >> 3) + i * (NT / 8);
    *reinterpret_cast<u32x4_t*>(lds + Lay<true>::off(r, tid & 7)) = reg[i];
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int K) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) load_unit(rs, ld, k0, K, i);
  }
  __device__ __forceinline__ void store(char* lds, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) store_unit(lds, tid, i);
  }
};

// M-major operand: element (r, k) at g[k * ld + r]; 16-byte chunks (8
// consecutive r of one k row) copied unchanged into the tile (see Lay<false>).
// Rows k >= kend read as zeros.
template <int R, int NT>
struct LoaderM {
  static constexpr int CPR = R / 8;  // chunks per k row
  static_assert(NT % CPR == 0 && BK * CPR % NT == 0, "k rows of chunks must split evenly over the threads");
  static constexpr int NCH = BK * CPR / NT;
  static constexpr int KSTEP = NT / CPR;  // k rows between a thread's chunks
  u32x4_t reg[NCH];
  uint32_t voff;  // this thread's chunk in k row krow (at k0 = 0)
  int krow, ch;
  __device__ __forceinline__ void init(int64_t ld, int row0, int tid) {
    krow = tid / CPR;
    ch = tid % CPR;
    voff = (uint32_t)(((int64_t)krow * ld + row0 + ch * 8) * 2);
  }
  // issue units: unit i is one chunk (load / store)
  static constexpr int NUNIT = NCH;
  __device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int kend, int i) {
    const int k = k0 + krow + i * KSTEP;
    const uint32_t oob = k < kend ? 0u : OOB_SHIFT;
    reg[i] = bload(rs, voff + (uint32_t)(((int64_t)(k0 + i * KSTEP) * ld) * 2) + oob);
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int kend) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) load_unit(rs, ld, k0, kend, i);
  }
  __device__ __forceinline__ void store_unit(char* lds, int tid, int i) {
    const int k = krow + i * KSTEP;
    *reinterpret_cast<u32x4_t*>(lds + Lay<false>::off<R>(k, ch * 8)) = reg[i];
  }
  __device__ __forceinline__ void store(char* lds, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) store_unit(lds, tid, i);
  }
};

// --- the MFMA kernel --------------------------------------------------------

// WGM x WGN waves, each owning a (BM / WGM) x (BN / WGN) block of 32x32 tiles;
// the k loop's schedule is described above it.
// GRP: 0 = one product; 1 = grouped, A rows contiguous per expert; 2 =
// grouped, A rows gathered through g_rows.
template <int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI, bool OUT_F32, int GRP>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma_kernel(GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1 && (EPI != EPI_SWIGLU || TN % 2 == 0), "bad wave tile");
  constexpr bool SW = (EPI == EPI_SWIGLU);
  constexpr int A_BUF = Lay<AK>::template BYTES<BM>, B_BUF = Lay<BKM>::template BYTES<BN>;
  extern __shared__ __align__(16) char smem[];
  // [A buffer 0][A buffer 1][B buffer 0][B buffer 1]
  char* const sA0 = smem;
  char* const sB0 = smem + 2 * A_BUF;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // tile order: contiguous ranges per XCD (workgroups are dealt round-robin
  // over the 8 XCDs), grouped 4 tile-rows at a time for L2 reuse, so that an
  // XCD's 32 concurrent tiles span 4 rows and 8 columns (groups of 8 rows, 4
  // columns: the Llama-8B-shaped step 0.37-0.40 ms longer; of 2 and 16 rows
  // longer still)
  int pid = blockIdx.x;
  const int ntiles = p.tiles_m * p.tiles_n;
  if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
  constexpr int GROUP = 4;
  const int in_group = GROUP * p.tiles_n;
  const int gid = pid / in_group;
  const int first_m = gid * GROUP;
  const int gsize = min(p.tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % in_group) % gsize;
  const int tile_n = (pid % in_group) / gsize;

  int m0 = tile_m * BM;
  const int n0 = SW ? tile_n * (BN / 2) : tile_n * BN;  // SwiGLU: F-column base

  if constexpr (GRP != 0) {
    // grouped: this tile covers rows [m0, m0 + BM) of expert e; C, C2, R and
    // the row factors are shifted to the expert's first row, B to its weights
    const int e = p.g_tile_e[tile_m];
    if (e < 0) return;  // idle tile (uniform over the workgroup, before any barrier)
    const int offe = p.g_off[e];
    m0 = p.g_tile_m0[tile_m];
    p.M = p.g_cnt[e];
    const size_t oes = OUT_F32 ? 4 : 2;
    p.C = (char*)p.C + (size_t)offe * p.ldc * oes;
    if (p.C2) p.C2 = (char*)p.C2 + (size_t)offe * p.ldc2 * 2;
    if (p.R) p.R = (const char*)p.R + (size_t)offe * p.ldr * oes;
    if (p.row_scale) p.row_scale += offe;
    p.B += (int64_t)e * p.b_stride;
    if constexpr (GRP == 1) {
      p.A += (int64_t)offe * p.lda;
      p.a_bytes -= (uint32_t)((int64_t)offe * p.lda * 2);
    } else {
      p.g_rows += offe;
    }
  }

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, p.b_bytes);
  constexpr int AMODE = GRP == 2 ? ROWS_GATHER : ROWS_CONTIG;
  std::conditional_t<AK, LoaderK<BM, AMODE, NT>, LoaderM<BM, NT>> la;
  constexpr bool RO = (EPI == EPI_ROPE);
  static_assert(!RO || (BKM && WN == 64 && !OUT_F32 && GRP == 0), "RoPE epilogue: K-major B, 64-column waves");
  std::conditional_t<BKM, LoaderK<BN, SW ? ROWS_SWIGLU : (RO ? ROWS_ROPE : ROWS_CONTIG), NT>, LoaderM<BN, NT>> lb;
  static_assert(GRP != 2 || AK, "gathered rows need a K-major A");
  if constexpr (AK) la.init(p.lda, m0, tid, 0, 1, p.g_rows, p.M);
  else la.init(p.lda, m0, tid);
  if constexpr (BKM) lb.init(p.ldb, n0, tid, RO ? p.N : p.F, WN);
  else lb.init(p.ldb, n0, tid);

  // k range of this split (the whole K unless the product is split along K)
  const int kbeg = blockIdx.y * p.kc;
  const int kend = min(p.K, kbeg + p.kc);
  auto load = [&](int k0) {
    la.load(ra, p.lda, k0, kend);
    lb.load(rb, p.ldb, k0, kend);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment rows of this lane
  const int arow = wm * WM + (lane & 31), brow = wn * WN + (lane & 31), kh = lane >> 5;
  // fragment q of k-substep ks, in the order the MFMAs consume them (A row
  // block 0, B row blocks 0 .. TN-1, then A row blocks 1 .. TM-1), so the
  // first MFMA of a substep waits for two reads only
  auto read_one = [&](const char* a_s, const char* b_s, int ks, int q, bf16x8_t (&af)[TM], bf16x8_t (&bfr)[TN]) {
    const int kc = ks * 2 + kh;
    if (q >= 1 && q <= TN) {
      if constexpr (BKM) bfr[q - 1] = *reinterpret_cast<const bf16x8_t*>(b_s + Lay<true>::off(brow + (q - 1) * 32, kc));
      else bfr[q - 1] = read_mm<BN>(b_s, wn * WN + (q - 1) * 32, ks, lane);
    } else {
      const int i = q == 0 ? 0 : q - TN;
      if constexpr (AK) af[i] = *reinterpret_cast<const bf16x8_t*>(a_s + Lay<true>::off(arow + i * 32, kc));
      else af[i] = read_mm<BM>(a_s, wm * WM + i * 32, ks, lane);
    }
  };

  // Software pipeline over 64-wide k tiles, two LDS buffers, one barrier per
  // tile. Entering tile kt: LDS[cur] holds tile kt, the registers hold its
  // substep-0 fragments, and the loaders' registers hold tile kt + 1 (loaded
  // one tile earlier). Substep s runs its MFMAs with substep s + 1's fragment
  // reads interleaved; substeps 0 to 2 also write tile kt + 1 into
  // LDS[cur ^ 1], each loader unit followed by its global load of tile
  // kt + 2, one unit every few MFMA slots (spread over the three substeps
  // rather than bunched into the first, which measured 1-11% faster). The
  // barrier closes substep 2, the last one that reads LDS[cur] and the last
  // that writes LDS[cur ^ 1]; after it tile kt + 1 is visible, so substep 3
  // reads tile kt + 1's substep-0 fragments under its MFMAs and no wave
  // waits on LDS at the top of the next tile. The next tile's stores (into
  // LDS[cur]) come after that same barrier. Prefetches past the end read
  // zeros (rows past the operand, the masked K tail) and are never consumed.
  constexpr int NKS = BK / 16;
  constexpr int NMF = TM * TN;  // MFMAs per k-substep
  constexpr int NRD = TM + TN;  // fragment reads per k-substep
  static_assert(NKS == 4, "the barrier placement assumes four substeps");
  static_assert(NRD <= NMF, "fewer MFMAs than fragment reads per substep");
  // With an M-major B operand in the eight-wave tile, the fragment reads are
  // spread evenly over the substep's MFMA slots instead of issued one per
  // slot from the first: it frees the registers that spilled there. The
  // K-major layouts keep the front-loaded reads, which spilled when spread,
  // and so does the four-wave tile.
  constexpr bool SPREAD_RD = !BKM && WGM * WGN == 8;
  // the loaders' issue units (A's, then B's) are spread over the MFMA slots of
  // the substeps before the barrier: slot ts = ks * NMF + t stores units
  // [ts * NU / NSL, (ts + 1) * NU / NSL) into the other buffer and reissues
  // their global loads for the tile after
  constexpr int NUA = decltype(la)::NUNIT, NU = NUA + decltype(lb)::NUNIT;
  constexpr int NSL = (NKS - 1) * NMF;
  const int nk = (kend - kbeg + BK - 1) / BK;
  load(kbeg);
  la.store(sA0, tid);
  lb.store(sB0, tid);
  load(kbeg + BK);
  __syncthreads();
  bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
  for (int q = 0; q < NRD; ++q) read_one(sA0, sB0, 0, q, af[0], bfr[0]);

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const char* a_s = sA0 + cur * A_BUF;
    const char* b_s = sB0 + cur * B_BUF;
    char* a_n = sA0 + (cur ^ 1) * A_BUF;
    char* b_n = sB0 + (cur ^ 1) * B_BUF;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int t = 0; t < NMF; ++t) {
        const int i = t / TN, j = t % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
        if constexpr (SPREAD_RD) {
          // slot t reads fragments [t * NRD / NMF, (t + 1) * NRD / NMF)
#pragma unroll
          for (int q = t * NRD / NMF; q < (t + 1) * NRD / NMF; ++q) {
            if (ks + 1 < NKS) read_one(a_s, b_s, ks + 1, q, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
            else read_one(a_n, b_n, 0, q, af[0], bfr[0]);
          }
        } else if (t < NRD) {
          if (ks + 1 < NKS) read_one(a_s, b_s, ks + 1, t, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
          else read_one(a_n, b_n, 0, t, af[0], bfr[0]);
        }
        if (ks < NKS - 1) {
          const int ts = ks * NMF + t;
#pragma unroll
          for (int u = ts * NU / NSL; u < (ts + 1) * NU / NSL; ++u) {
            if (u < NUA) {
              la.store_unit(a_n, tid, u);
              la.load_unit(ra, p.lda, kbeg + (kt + 2) * BK, kend, u);
            } else {
              lb.store_unit(b_n, tid, u - NUA);
              lb.load_unit(rb, p.ldb, kbeg + (kt + 2) * BK, kend, u - NUA);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ks == 2) __syncthreads();
    }
  }

  // --- epilogue. The MFMA result gives a lane one column of each 32x32 tile
  // (rows 8 (r / 4) + 4 (lane / 32) + r % 4 in register r), so storing it
  // directly takes one 2- or 4-byte access per element and lane. Instead each
  // wave passes its block through LDS, 32 rows at a time, in a region of its
  // own: it writes the 32 x WN accumulators and reads them back as rows of 4
  // consecutive columns per lane, so every global load and store of the
  // epilogue moves 4 elements (one 8- or 16-byte access when p.vec allows).
  // Rows of the staging block are WN + 8 floats apart, so the two halves of a
  // wave's writes (rows 4 apart) fall in different banks.
  const int lc = lane & 31, lr = (lane >> 5) * 4;
  if constexpr (OUT_F32 && EPI == EPI_STORE) {
    // Plain fp32 stores go out directly: each half-wave writes a whole
    // 128-byte row segment per instruction, and the store burst is bound by
    // HBM writes either way; the staging pass measured 1-3% slower here.
    // They are non-temporal (these outputs, logits and weight gradients, are
    // next read by another kernel from HBM, not from this XCD's L2): 0.25 ms
    // off the Llama-8B-shaped step, three interleaved rounds.
    if (!p.accumulate) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn * WN + j * 32 + lc;
          if (n >= p.N) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lr + (r & 3);
            if (m >= p.M) continue;
            float v = acc[i][j][r] * p.alpha;
            if (p.row_scale) v *= p.row_scale[m];
            __builtin_nontemporal_store(v, reinterpret_cast<float*>(p.C) + blockIdx.y * p.c_split + (int64_t)m * p.ldc + n);
          }
        }
      return;
    }
  }
  __syncthreads();  // the k loop's last LDS reads are done in every wave
  constexpr int CS = WN + 8;
  static_assert(WGM * WGN * 32 * CS * 4 <= 2 * (A_BUF + B_BUF), "the staging blocks must fit in the k loop's LDS");
  float* const stg = reinterpret_cast<float*>(smem) + wave * 32 * CS;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stg[(8 * (r >> 2) + lr + (r & 3)) * CS + j * 32 + lc] = acc[i][j][r];
    const int mb = m0 + wm * WM + i * 32;  // first row of this block
    if constexpr (EPI == EPI_ROPE || EPI == EPI_SWIGLU) {
      // two halves of WN / 2 columns each: RoPE's first and second members of
      // the rotation pairs (dims dl and dl + 64 of one head), SwiGLU's gate
      // and up pre-activations of the same output column
      constexpr int HW = WN / 2, LPR = HW / 4, RPI = 64 / LPR;
      const int c4 = 4 * (lane % LPR);
#pragma unroll
      for (int q = 0; q < 32 / RPI; ++q) {
        const int row = lane / LPR + q * RPI, m = mb + row;
        const float4 a4 = *reinterpret_cast<const float4*>(stg + row * CS + c4);
        const float4 b4 = *reinterpret_cast<const float4*>(stg + row * CS + HW + c4);
        float a[4] = {a4.x, a4.y, a4.z, a4.w}, bb[4] = {b4.x, b4.y, b4.z, b4.w};
        if (m >= p.M) continue;
        if constexpr (EPI == EPI_ROPE) {
          bf16* c = reinterpret_cast<bf16*>(p.C);
          const int head = (n0 >> 7) + (wn >> 1);
          const int dl = (wn & 1) * 32 + c4;
          const int col = head * 128 + dl;
          if (col >= p.N) continue;  // whole heads: the four dims are in range together
          if (p.R) {  // an addend of the same layout (the LoRA deltas), before the rotation
            const bf16* rr = reinterpret_cast<const bf16*>(p.R) + (int64_t)m * p.ldr + col;
            float x[4], y[4];
            ld4(rr, 4, p.vec, x);
            ld4(rr + 64, 4, p.vec, y);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] += x[e];
              bb[e] += y[e];
            }
          }
          if (head < p.rope_heads) {
            const float2* tab = p.rope_tab + (m % p.rope_seq) * 64 + dl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float2 cs = tab[e];
              const float l2 = a[e] * cs.x - bb[e] * cs.y;
              bb[e] = bb[e] * cs.x + a[e] * cs.y;
              a[e] = l2;
            }
          }
          st4(c + (int64_t)m * p.ldc + col, 4, p.vec, a);
          st4(c + (int64_t)m * p.ldc + col + 64, 4, p.vec, bb);
        } else {
          const int f = n0 + wn * HW + c4;
          if (f >= p.F) continue;
          const int cnt = min(4, p.F - f);
          float mo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) mo[e] = silu_f(a[e]) * bb[e];
          if (!p.skip_c) {
            bf16* gu = reinterpret_cast<bf16*>(p.C) + (int64_t)m * p.ldc;
            st4(gu + f, cnt, p.vec, a);
            st4(gu + p.F + f, cnt, p.vec, bb);
          }
          st4(reinterpret_cast<bf16*>(p.C2) + (int64_t)m * p.ldc2 + f, cnt, p.vec, mo);
        }
      }
    } else {
      constexpr int LPR = WN / 4, RPI = 64 / LPR;
      const int c4 = 4 * (lane % LPR);
      const int n = n0 + wn * WN + c4;
#pragma unroll
      for (int q = 0; q < 32 / RPI; ++q) {
        const int row = lane / LPR + q * RPI, m = mb + row;
        const float4 a4 = *reinterpret_cast<const float4*>(stg + row * CS + c4);
        if (m >= p.M || n >= p.N) continue;
        const int cnt = min(4, p.N - n);
        float v[4] = {a4.x * p.alpha, a4.y * p.alpha, a4.z * p.alpha, a4.w * p.alpha};
        if (p.row_scale) {
          const float rs = p.row_scale[m];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= rs;
        }
        if constexpr (EPI == EPI_SWIGLU_BWD) {
          const bf16* gu = reinterpret_cast<const bf16*>(p.R) + (int64_t)m * p.ldr;
          float g[4], u[4], dg[4], du[4];
          ld4(gu + n, cnt, p.vec, g);
          ld4(gu + p.F + n, cnt, p.vec, u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sg = 1.f / (1.f + __expf(-g[e]));
            dg[e] = v[e] * u[e] * sg * (1.f + g[e] * (1.f - sg));
            du[e] = v[e] * g[e] * sg;
          }
          bf16* dgu = reinterpret_cast<bf16*>(p.C) + (int64_t)m * p.ldc;
          st4(dgu + n, cnt, p.vec, dg);
          st4(dgu + p.F + n, cnt, p.vec, du);
        } else if constexpr (OUT_F32) {
          float* c = reinterpret_cast<float*>(p.C) + blockIdx.y * p.c_split + (int64_t)m * p.ldc + n;
          if (EPI == EPI_RESID) {
            float x[4];
            ld4(reinterpret_cast<const float*>(p.R) + (int64_t)m * p.ldr + n, cnt, p.vec, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += x[e];
          }
          if (p.accumulate) {
            float o[4];
            ld4(c, cnt, p.vec, o);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[e] + v[e];
          }
          st4(c, cnt, p.vec, v);
        } else {
          if (EPI == EPI_RESID) {
            float x[4];
            ld4(reinterpret_cast<const bf16*>(p.R) + (int64_t)m * p.ldr + n, cnt, p.vec, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += x[e];
          }
          st4(reinterpret_cast<bf16*>(p.C) + (int64_t)m * p.ldc + n, cnt, p.vec, v);
        }
      }
    }
  }
}

// --- the generic kernel -----------------------------------------------------

template <class TI>
struct SimpleParams {
  int M, N, K;
  const TI* A; int64_t sam, sak;
  const TI* B; int64_t sbn, sbk;
};

// 64x64 output tile, 16x16 threads with 4x4 outputs each; writes fp32 acc
// through the epilogue functor
template <class TI, class TO, int EPI>
__global__ __launch_bounds__(256) void gemm_simple_kernel(SimpleParams<TI> p, TO* C, int64_t ldc,
                                                          const TO* R, int64_t ldr, int accumulate, float alpha) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    for (int i = threadIdx.x; i < 1024; i += 256) {
      int kk = i & 15, mm = i >> 4;
      int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < p.M && k < p.K) ? to_f(p.A[m * p.sam + k * p.sak]) : 0.f;
      int n = n0 + mm;
      Bs[kk][mm] = (n < p.N && k < p.K) ? to_f(p.B[n * p.sbn + k * p.sbk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m >= p.M || n >= p.N) continue;
      float v = acc[i][j] * alpha;
      if (EPI == EPI_RESID) v += to_f(R[(int64_t)m * ldr + n]);
      TO* c = C + (int64_t)m * ldc + n;
      if (accumulate) v += to_f(*c);
      *c = from_f<TO>(v);
    }
}

template <class TI, class TO, int EPI>
rp_status launch_simple(const GemmDesc& d, void* C, int64_t ldc, hipStream_t s) {
  SimpleParams<TI> p;
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.A = reinterpret_cast<const TI*>(d.A);
  p.sam = d.a_kmajor ? d.lda : 1; p.sak = d.a_kmajor ? 1 : d.lda;
  p.B = reinterpret_cast<const TI*>(d.B);
  p.sbn = d.b_kmajor ? d.ldb : 1; p.sbk = d.b_kmajor ? 1 : d.ldb;
  dim3 grid(cdiv(d.N, 64), cdiv(d.M, 64));
  TraceScope ts(s, "gemm_simple_kernel", 2.0 * d.M * d.N * d.K, 0.0);
  RP_LAUNCH((gemm_simple_kernel<TI, TO, EPI>), grid, dim3(256), 0, s, p,
            reinterpret_cast<TO*>(C), ldc, reinterpret_cast<const TO*>(d.R), d.ldr,
            (int)d.accumulate, d.alpha);
  return RP_OK;
}

template <class TI>
rp_status gemm_simple(const GemmDesc& d, hipStream_t s) {
  const bool of32 = d.out_dtype == RP_DTYPE_F32;
  switch (d.epi) {
    case EPI_STORE:
      if (of32) return launch_simple<TI, float, EPI_STORE>(d, d.C, d.ldc, s);
      return launch_simple<TI, bf16, EPI_STORE>(d, d.C, d.ldc, s);
    case EPI_RESID:
      if (of32) return launch_simple<TI, float, EPI_RESID>(d, d.C, d.ldc, s);
      return launch_simple<TI, bf16, EPI_RESID>(d, d.C, d.ldc, s);
    case EPI_SWIGLU: {
      // gu = A B^T into C, then m = silu(g) * u
      if (of32) RP_TRY((launch_simple<TI, float, EPI_STORE>(d, d.C, d.ldc, s)));
      else RP_TRY((launch_simple<TI, bf16, EPI_STORE>(d, d.C, d.ldc, s)));
      RP_CHECK(d.ldc == d.N && d.ldc2 == d.N / 2, RP_ERR_UNSUPPORTED, "swiglu: packed rows required");
      return swiglu_fwd(d.out_dtype, d.C, d.C2, d.M, d.N / 2, s);
    }
    case EPI_SWIGLU_BWD: {
      RP_CHECK(d.tmp != nullptr, RP_ERR_INVALID, "swiglu bwd: fp32 scratch missing");
      GemmDesc e = d;
      e.accumulate = false;
      RP_TRY((launch_simple<TI, float, EPI_STORE>(e, d.tmp, d.N, s)));
      RP_CHECK(d.ldc == 2 * d.N && d.ldr == 2 * d.N, RP_ERR_UNSUPPORTED, "swiglu bwd: packed rows required");
      return swiglu_bwd(d.out_dtype, d.tmp, d.R, d.C, d.M, d.N, s);
    }
  }
  set_error("gemm: unknown epilogue %d", d.epi);
  return RP_ERR_INVALID;
}

// --- MFMA dispatch ------------------------------------------------------------

// bytes spanned by an operand of `rows` x `k` stored with leading dimension ld
inline uint64_t operand_bytes(bool kmajor, int64_t rows, int64_t k, int64_t ld) {
  if (rows == 0 || k == 0) return 0;
  return (uint64_t)(kmajor ? (rows - 1) * ld + k : (k - 1) * ld + rows) * 2;
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI, bool OF32, int GRP = 0>
rp_status launch_mfma(const GemmDesc& d, hipStream_t s) {
  GemmParams p{};
  p.M = d.M; p.N = d.N; p.K = d.K;
  p.A = reinterpret_cast<const bf16*>(d.A); p.lda = d.lda;
  p.B = reinterpret_cast<const bf16*>(d.B); p.ldb = d.ldb;
  p.C = d.C; p.ldc = d.ldc;
  p.R = d.R; p.ldr = d.ldr;
  p.C2 = d.C2; p.ldc2 = d.ldc2;
  p.skip_c = EPI == EPI_SWIGLU && d.c_unused ? 1 : 0;
  p.accumulate = d.accumulate ? 1 : 0;
  p.alpha = d.alpha;
  p.kc = d.K;
  p.c_split = 0;
  int splits = 1;
  if (d.split_k > 1) {
    // split K into ranges of whole 64-wide steps; each writes an fp32 partial
    p.kc = (int)(cdiv(cdiv(d.K, d.split_k), BK) * BK);
    splits = (int)cdiv(d.K, p.kc);
    p.C = d.partial;
    p.ldc = d.N;
    p.c_split = (int64_t)d.M * d.N;
    p.accumulate = 0;
  }
  p.F = EPI == EPI_SWIGLU ? d.N / 2 : (EPI == EPI_SWIGLU_BWD ? d.N : 0);
  p.tiles_m = (int)cdiv(d.M, BM);
  p.tiles_n = EPI == EPI_SWIGLU ? (int)cdiv(d.N / 2, BN / 2) : (int)cdiv(d.N, BN);
  p.row_scale = d.row_scale;
  p.rope_tab = d.rope_tab;
  p.rope_seq = d.rope_seq;
  p.rope_heads = d.rope_heads;
  uint64_t ab = operand_bytes(AK, d.M, d.K, d.lda), bb = operand_bytes(BKM, d.N, d.K, d.ldb);
  if constexpr (GRP != 0) {
    const GemmGroup& g = *d.group;
    p.tiles_m = g.max_tiles_m;
    p.g_tile_e = g.tile_e;
    p.g_tile_m0 = g.tile_m0;
    p.g_off = g.off;
    p.g_cnt = g.cnt;
    p.g_rows = g.rows;
    p.b_stride = g.b_stride;
    ab = operand_bytes(AK, g.a_rows, d.K, d.lda);  // the whole operand: rows are per expert
    // d.N x d.K is one expert's B
  }
  RP_CHECK(ab < (1ull << 31) && bb < (1ull << 31), RP_ERR_UNSUPPORTED,
           "gemm(bf16): each operand must span less than 2 GiB");
  p.a_bytes = (uint32_t)ab;
  p.b_bytes = (uint32_t)bb;
  {
    // the epilogue's four-element accesses: row strides and the column offset
    // F in multiples of 4 elements, bases aligned to 4 elements
    const size_t ce = OF32 ? 4 : 2;
    const size_t re = EPI == EPI_RESID ? ce : 2;
    auto al = [](const void* q, size_t b) { return reinterpret_cast<uintptr_t>(q) % b == 0; };
    bool v = p.ldc % 4 == 0 && al(p.C, 4 * ce) && p.c_split % 4 == 0 && p.F % 4 == 0;
    if (p.R) v = v && p.ldr % 4 == 0 && al(p.R, 4 * re);
    if (p.C2) v = v && p.ldc2 % 4 == 0 && al(p.C2, 8);
    p.vec = v ? 1 : 0;
  }
  const size_t lds = 2 * ((size_t)Lay<AK>::template BYTES<BM> + (size_t)Lay<BKM>::template BYTES<BN>);
  static bool attr_set = false;  // one instantiation per template: set once
  if (!attr_set) {
    RP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mfma_kernel<BM, BN, WGM, WGN, AK, BKM, EPI, OF32, GRP>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    attr_set = true;
  }
  const int64_t nt = (int64_t)p.tiles_m * p.tiles_n;
  char name[96];
  snprintf(name, sizeof(name), "gemm_mfma_kernel<%d, %d, %d, %d, %d, %d, %d, %d, %d>", BM, BN, WGM, WGN, (int)AK,
           (int)BKM, EPI, (int)OF32, GRP);
  // grouped products: d.M is the total of the experts' rows
  TraceScope ts(s, name, 2.0 * d.M * d.N * d.K, 0.0);
  RP_LAUNCH((gemm_mfma_kernel<BM, BN, WGM, WGN, AK, BKM, EPI, OF32, GRP>), dim3((unsigned)nt, (unsigned)splits),
            dim3(64 * WGM * WGN), lds, s, p);
  if (splits > 1) return splitk_reduce(d.partial, splits, d.M, d.N, reinterpret_cast<float*>(d.C), d.ldc, d.accumulate, s);
  return RP_OK;
}

template <int BM, int BN, int WGM, int WGN, int EPI, bool OF32>
rp_status dispatch_layout(const GemmDesc& d, hipStream_t s) {
  if constexpr (BM == 256 && BN == 256 && WGM == 2 && WGN == 4 && EPI != EPI_SWIGLU) {
    // M-major A, K-major B: 64 x 128 wave tiles, so that the operand whose
    // fragments take two transposing reads each is the one with fewer
    // fragments per wave
    if (!d.a_kmajor && d.b_kmajor) return launch_mfma<BM, BN, 4, 2, false, true, EPI, OF32>(d, s);
  }
  if (d.a_kmajor && d.b_kmajor) return launch_mfma<BM, BN, WGM, WGN, true, true, EPI, OF32>(d, s);
  if (d.a_kmajor && !d.b_kmajor) return launch_mfma<BM, BN, WGM, WGN, true, false, EPI, OF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor) return launch_mfma<BM, BN, WGM, WGN, false, false, EPI, OF32>(d, s);
  return launch_mfma<BM, BN, WGM, WGN, false, true, EPI, OF32>(d, s);
}

template <int BM, int BN, int WGM, int WGN>
rp_status dispatch_epi(const GemmDesc& d, hipStream_t s) {
  const bool of32 = d.out_dtype == RP_DTYPE_F32;
  switch (d.epi) {
    case EPI_STORE:
      return of32 ? dispatch_layout<BM, BN, WGM, WGN, EPI_STORE, true>(d, s)
                  : dispatch_layout<BM, BN, WGM, WGN, EPI_STORE, false>(d, s);
    case EPI_RESID:
      return of32 ? dispatch_layout<BM, BN, WGM, WGN, EPI_RESID, true>(d, s)
                  : dispatch_layout<BM, BN, WGM, WGN, EPI_RESID, false>(d, s);
    case EPI_SWIGLU:
      RP_CHECK(d.b_kmajor && !of32, RP_ERR_UNSUPPORTED, "swiglu epilogue: K-major bf16 only");
      return dispatch_layout<BM, BN, WGM, WGN, EPI_SWIGLU, false>(d, s);
    case EPI_SWIGLU_BWD:
      RP_CHECK(!of32, RP_ERR_UNSUPPORTED, "swiglu bwd epilogue: bf16 only");
      return dispatch_layout<BM, BN, WGM, WGN, EPI_SWIGLU_BWD, false>(d, s);
    case EPI_ROPE:
      RP_CHECK(!of32 && d.a_kmajor && d.b_kmajor, RP_ERR_UNSUPPORTED, "rope epilogue: K-major bf16 only");
      if constexpr (BN / WGN == 64) return launch_mfma<BM, BN, WGM, WGN, true, true, EPI_ROPE, false>(d, s);
      set_error("rope epilogue: needs 64-column wave tiles");
      return RP_ERR_UNSUPPORTED;
  }
  set_error("gemm: unknown epilogue %d", d.epi);
  return RP_ERR_INVALID;
}

}  // namespace

// both operands M-major: K is a row index of each, any value works
#define K_MULT_FREE(d) (!(d).a_kmajor && !(d).b_kmajor)

rp_status gemm_validate(const GemmDesc& d) {
  RP_CHECK(d.M >= 0 && d.N >= 0 && d.K >= 0, RP_ERR_INVALID, "gemm: negative size");
  RP_CHECK(d.A && d.B && d.C, RP_ERR_INVALID, "gemm: null operand");
  RP_CHECK(d.lda >= (d.a_kmajor ? d.K : d.M) && d.ldb >= (d.b_kmajor ? d.K : d.N), RP_ERR_INVALID,
           "gemm: leading dimension too small");
  if (d.in_dtype == RP_DTYPE_BF16 && !d.force_simple) {
    // 16-byte chunks run along K for K-major operands (a chunk may not
    // straddle K) and along M / N for M-major ones (rows start 16-byte aligned)
    RP_CHECK((K_MULT_FREE(d) || d.K % 8 == 0) && d.lda % 8 == 0 && d.ldb % 8 == 0, RP_ERR_UNSUPPORTED,
             "gemm(bf16): leading dimensions, and K when an operand is K-major, must be multiples of 8");
    RP_CHECK(((uintptr_t)d.A & 15) == 0 && ((uintptr_t)d.B & 15) == 0, RP_ERR_INVALID,
             "gemm(bf16): operands must be 16-byte aligned");
    if (d.epi == EPI_SWIGLU) RP_CHECK(d.N % 2 == 0, RP_ERR_INVALID, "swiglu: N must be even");
  }
  if (d.epi == EPI_RESID || d.epi == EPI_SWIGLU_BWD) RP_CHECK(d.R, RP_ERR_INVALID, "gemm: missing R");
  if (d.epi == EPI_SWIGLU) RP_CHECK(d.C2, RP_ERR_INVALID, "gemm: missing C2");
  if (d.epi == EPI_ROPE)
    RP_CHECK(d.in_dtype == RP_DTYPE_BF16 && d.out_dtype == RP_DTYPE_BF16 && !d.force_simple && d.a_kmajor &&
                 d.b_kmajor && d.rope_tab && d.rope_seq > 0 && d.N % 128 == 0 && d.rope_heads >= 0 &&
                 d.split_k <= 1 && !d.accumulate && d.alpha == 1.f,
             RP_ERR_UNSUPPORTED, "gemm: the RoPE epilogue needs bf16 K-major operands, heads of 128 and the table");
  RP_CHECK(!d.accumulate || d.out_dtype == RP_DTYPE_F32, RP_ERR_INVALID,
           "gemm: accumulation needs an fp32 output");
  if (d.split_k > 1)
    RP_CHECK(d.in_dtype == RP_DTYPE_BF16 && d.out_dtype == RP_DTYPE_F32 && d.epi == EPI_STORE && d.partial &&
                 d.partial_bytes >= splitk_bytes(d.M, d.N, d.K, d.split_k),
             RP_ERR_INVALID, "gemm: split-K needs bf16 operands, a plain fp32 store and its partial scratch");
  RP_CHECK(d.alpha == 1.f || d.epi == EPI_STORE || d.epi == EPI_RESID, RP_ERR_INVALID,
           "gemm: alpha applies to the store and residual epilogues only");
  return RP_OK;
}

rp_status gemm(const GemmDesc& dd, hipStream_t s) {
  GemmDesc d = dd;
  if (d.split_k == 0) {
    // automatic split-K for products with few output tiles and a long K (the
    // LoRA adapter gradients): enough ranges to give ~512 workgroups
    d.split_k = 1;
    const int64_t tiles = cdiv(d.M, 128) * cdiv(d.N, 128);
    if (d.in_dtype == RP_DTYPE_BF16 && d.out_dtype == RP_DTYPE_F32 && d.epi == EPI_STORE && d.partial &&
        tiles < 128 && d.K >= 1024) {
      int sk = (int)std::min<int64_t>(cdiv(512, tiles), d.K / 256);
      while (sk > 1 && splitk_bytes(d.M, d.N, d.K, sk) > d.partial_bytes) --sk;
      d.split_k = std::max(sk, 1);
    }
  }
  RP_TRY(gemm_validate(d));
  if (d.M == 0 || d.N == 0) return RP_OK;
  if (d.K == 0) {
    RP_CHECK(d.epi == EPI_STORE, RP_ERR_UNSUPPORTED, "gemm: K == 0 only for plain stores");
    if (d.accumulate) return RP_OK;
    // C = 0 row by row
    for (int m = 0; m < d.M; ++m)
      RP_TRY(fill_zero((char*)d.C + (size_t)m * d.ldc * dtype_size(d.out_dtype),
                       (size_t)d.N * dtype_size(d.out_dtype), s));
    return RP_OK;
  }
  if (d.in_dtype == RP_DTYPE_F32) return gemm_simple<float>(d, s);
  if (d.force_simple) return gemm_simple<bf16>(d, s);
  if (d.split_k > 1) return dispatch_epi<128, 128, 2, 2>(d, s);
  const int64_t n_eff = d.epi == EPI_SWIGLU ? d.N / 2 : d.N;
  const int64_t big = cdiv(d.M, 256) * cdiv(n_eff, d.epi == EPI_SWIGLU ? 128 : 256);
  if (big < 240) return dispatch_epi<128, 128, 2, 2>(d, s);
  return dispatch_epi<256, 256, 2, 4>(d, s);
}

rp_status gemm_grouped(const GemmDesc& d, hipStream_t s) {
  RP_CHECK(d.group && d.in_dtype == RP_DTYPE_BF16 && d.out_dtype == RP_DTYPE_BF16 && d.split_k == 1 && !d.accumulate,
           RP_ERR_INVALID, "gemm_grouped: bf16 in/out, no split, no accumulation");
  RP_CHECK(d.K % 8 == 0 && d.lda % 8 == 0 && d.ldb % 8 == 0 && ((uintptr_t)d.A & 15) == 0 &&
               ((uintptr_t)d.B & 15) == 0 && d.a_kmajor && d.A && d.B && d.C,
           RP_ERR_INVALID, "gemm_grouped: K-major A, aligned operands");
  if (d.M == 0 || d.N == 0 || d.group->max_tiles_m == 0) return RP_OK;
  const bool gather = d.group->rows != nullptr;
  if (d.epi == EPI_SWIGLU && d.b_kmajor)
    return gather ? launch_mfma<GROUP_BM, 256, 2, 4, true, true, EPI_SWIGLU, false, 2>(d, s)
                  : launch_mfma<GROUP_BM, 256, 2, 4, true, true, EPI_SWIGLU, false, 1>(d, s);
  if (d.epi == EPI_STORE && d.b_kmajor && !gather)
    return launch_mfma<GROUP_BM, 256, 2, 4, true, true, EPI_STORE, false, 1>(d, s);
  if (d.epi == EPI_SWIGLU_BWD && !d.b_kmajor && gather)
    return launch_mfma<GROUP_BM, 256, 2, 4, true, false, EPI_SWIGLU_BWD, false, 2>(d, s);
  if (d.epi == EPI_STORE && !d.b_kmajor && !gather)
    return launch_mfma<GROUP_BM, 256, 2, 4, true, false, EPI_STORE, false, 1>(d, s);
  set_error("gemm_grouped: unsupported combination (epilogue %d, B %s, A %s)", d.epi,
            d.b_kmajor ? "K-major" : "M-major", gather ? "gathered" : "contiguous");
  return RP_ERR_UNSUPPORTED;
}

size_t splitk_bytes(int64_t M, int64_t N, int64_t K, int split_k) {
  if (split_k <= 1) return 0;
  const int64_t kc = cdiv(cdiv(K, split_k), BK) * BK;
  return (size_t)cdiv(K, kc) * M * N * sizeof(float);
}

}  // namespace rp
