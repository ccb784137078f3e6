// Split-KV tree-masked attention for CDNA4 (gfx950): verification over the
// full cache and drafting over the partial cache share these kernels.
//
// What is computed (TokenSwift summary §3.1 with Figure 2, §3.3, Appendix E
// "Tree-Based Attention"): for every query head h of KV head g and every tree
// node i, softmax-weighted values over the committed rows plus the node's own
// ancestors-or-self among the tree rows appended after the context.
//
// Work decomposition
//   grid.x  = cache chunk ("split") of one KV head, grid.y = KV head,
//   grid.z  = block of query rows when a group has more rows than one
//             workgroup holds.
//   The M = G*T query rows of a KV head (G query heads x T tree nodes) are
//   cut into 16-row MFMA tiles; the RG x PG waves of a workgroup split them
//   into RG row groups of TPW row tiles and each K/V tile into PG groups of 32
//   positions, so the K/V tile staged in LDS once serves every head of the
//   group and every node. Per K/V tile of TN = 32 * PG positions:
//     S^T = K Q^T     v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q
//                     from LDS or registers); a lane holds 4 positions of one
//                     query row, so row statistics are lane-local plus two
//                     cross-lane permutes.
//     online softmax  base-2, scale folded into one FMA before exp2, lazy
//                     rescaling of the running max.
//     O^T += V^T P^T  v_mfma_f32_16x16x32_f16; P is packed to f16 straight
//                     from the S^T accumulators (no shuffles); V^T comes from
//                     LDS with ds_read_b64_tr_b16, converted bf16 -> f16 in
//                     registers (or once per tile in LDS when three or more
//                     row groups would each convert it).
//   All global reads are asynchronous copies into LDS (the first K tile, the
//   queries and the tree's ancestor words, then a STAGES-deep K/V ring).
//   The eight-wave forms without score sums take one barrier per tile (K of
//   the tile landed and the previous tile done everywhere) and a count in LDS
//   of the landed or converted V tile before P V; the others take two (K
//   landed / previous P V done, and V landed / K reads done).
//   Splits write (max, sum, normalised output) partials, the output in f16
//   (half the bytes of the split's stores and the combine's reads); a combine
//   kernel merges them with the log-sum-exp rule. A single split normalises
//   in place.
//
// Fused grouped scores (optional, TokenSwift summary §3.3 "Dynamic KV Cache
// Management"): the importance score of a committed row under GQA is the sum
// of its query-key products over the group's query heads and tree nodes. The
// raw S^T tile already holds every one of those products, so a workgroup that
// holds all query rows of its KV head sums each tile over its rows (lanes,
// then row tiles, then row groups through LDS) and writes sigma for the
// tile's committed rows: no second pass over K.
#include "ts_device.h"
#include "ts_internal.h"

#include <cmath>
#include <type_traits>

namespace ts {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D, int RG, int PG, int TPW, int STAGES, bool SCORE = false>
struct Cfg {
  static constexpr int NCH = D / 8;                       // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                      // bytes per staged row
  static constexpr int NW = RG * PG;                      // waves
  static constexpr int NT = NW * 64;                      // threads
  static constexpr int KSTEPS = D / 32;                   // MFMA k-steps over channels
  static constexpr int TN = 32 * PG;                      // positions per KV tile (32 per wave)
  static constexpr int CT = D / 16;                       // 16-channel output tiles
  static constexpr int TILE_BYTES = TN * ROWB;            // per tensor
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;      // K then V
  static constexpr int ROWS_PER_DMA = 1024 / ROWB;        // one wave-wide 16 B/lane DMA = 1 KB
  static constexpr int LANES_PER_ROW = ROWB / 16;
  static constexpr int DMA_PER_TENSOR = TN / ROWS_PER_DMA;
  static constexpr int DMA_PER_STAGE = 2 * DMA_PER_TENSOR;
  // Copies are issued by the first NI waves. With two waves per SIMD the
  // first four (one per SIMD) take them all: a copy's issue can stall for
  // tens of cycles while the memory pipeline is full, and the waves created
  // first win the SIMD's issue arbitration and arrive at every barrier early,
  // so those stalls stay off the later waves' path.
  static constexpr int NI = NW >= 8 ? NW / 2 : NW;
  static constexpr int DMA_MIN_PER_WAVE = DMA_PER_STAGE / NI;  // every issuing wave issues at least this many
  static constexpr int DMA_T_PER_WAVE = (DMA_PER_TENSOR + NI - 1) / NI;  // per tensor, at most
  static constexpr int DMA_T_MIN = DMA_PER_TENSOR / NI;                  // per tensor, at least
  static constexpr int ROWS_PER_BLOCK = RG * TPW * 16;
  static constexpr int KV_BYTES = STAGES * STAGE_BYTES;
  static constexpr int Q_BYTES = ROWS_PER_BLOCK * ROWB;    // the block's query rows
  // 8-wave shapes with few row tiles per wave keep their query fragments in
  // registers after the first tile (fewer LDS reads per tile); the others
  // read them from LDS each tile (registers are short).
  static constexpr bool Q_REG = NW >= 8 && TPW <= 3;
  // With three or more row groups, each V fragment would be converted bf16 ->
  // f16 by that many waves: convert the tile once in LDS instead (measured:
  // T = 64 shapes -6% with every wave converting a share and a barrier before
  // the softmax, a further -3% with the issuing waves converting and the
  // barrier after the softmax, and -4% more with a counter of converted
  // shares in place of that barrier; at RG = 2 converting in registers is
  // faster).
  static constexpr bool V_SHARED = RG >= 3;
  static constexpr int ANC_BYTES = 2048;  // ancestor words of the tree nodes (two 64-lane copies)
  // fused scores: the row sums of row groups 1.. for row group 0 (32 positions per wave)
  static constexpr int SC_BYTES = SCORE && RG > 1 ? (RG - 1) * PG * 32 * 4 : 0;
  // At the end of a split each wave keeps the CT / PG channel tiles it merges
  // and parks the others (and its m, l) for the waves that merge them.
  static constexpr int CT_OUT = PG > 1 ? CT - CT / PG : CT;
  static constexpr int MSLOT = 64 * CT_OUT * 16 + 2 * 16 * 4;   // one wave's parked O^T of a row tile + m, l
  static constexpr int MERGE_BYTES = PG * RG * MSLOT;
  // count of the V tile's converted shares (shared conversion) or landed
  // copies (two row groups without score sums), read by every wave before P V
  static constexpr int CNT_BYTES = V_SHARED || (!SCORE && NW >= 8) ? 16 : 0;
  static constexpr int LDS_BYTES = KV_BYTES + Q_BYTES + ANC_BYTES + SC_BYTES + CNT_BYTES;
  // row tiles merged per round at the end of a split (all of LDS is free then)
  // (the score slots stay out of it: row group 0 may still read them)
  static constexpr int MERGE_LDS = LDS_BYTES - SC_BYTES - CNT_BYTES;
  static constexpr int MERGE_RT = MERGE_LDS / (NW * MSLOT) < TPW ? MERGE_LDS / (NW * MSLOT) : TPW;
  static_assert(MERGE_BYTES <= KV_BYTES, "split-local merge reuses the K/V ring");
  static_assert(CT % PG == 0, "merge splits the channel tiles evenly over position groups");
  static_assert(DMA_MIN_PER_WAVE >= 1, "every issuing wave takes part in staging");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
};

// Reference-max slack of the online softmax, in log2 units.
constexpr float LAZY_LOG2 = 8.0f;
// Running-max start: finite, so no -inf special cases (masked scores are -inf
// and give exp2(-inf) = 0; a row with any visible score moves the max).
constexpr float NEG_BIG = -1.0e30f;

// max(a, b, c) in one v_max3_f32. Scores are finite or -inf (never NaN), so
// the IEEE-mode quieting that fmaxf would add before every max is not needed.
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Lane-local max of the 8 scores a lane holds for one row.
__device__ inline float lane_max8(const f32x4& x, const f32x4& y) {
  return max3(max3(x[0], x[1], x[2]), max3(x[3], y[0], y[1]), max3(y[2], y[3], y[3]));
}

// Max over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 row-swap permutes: VALU only, no LDS round trip. With both operands
// holding x, permlane16_swap leaves rows (0,0,2,2) in one result and (1,1,3,3)
// in the other; permlane32_swap does the same for the two halves.
__device__ inline float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ inline float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// bf16 pair (low, high halves of a 32-bit word) -> f16 pair in one
// v_cvt_pk_f16_f32 (round to nearest even). Exact for bf16 values in the f16
// normal range; magnitudes of 65536 and up (the next bf16 value past the f16
// maximum) become +-inf, so such a V value makes the output rows that see it
// non-finite instead of silently clamped.
__device__ inline unsigned int bf16x2_to_f16x2(unsigned int w) {
  const f2v x = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(x, f16x2));
}

template <int CTRL>
__device__ inline float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sums each of x[0..7] over the 16 lanes of a DPP row and leaves sum j =
// 4*b3 + 2*b2 + b1 in the lanes whose index in the row has bits (b3, b2, b1)
// (lanes 2m and 2m+1 hold the same value). Reduce-scatter by exchange with
// partners at xor 8, 7 (row_half_mirror), 2 and 1: each step adds the half
// the lane keeps to the partner's copy of it, so 4 + 2 + 1 + 1 adds in place
// of 8 x 4 for full row sums.
__device__ inline float row16_scatter8(const float (&x)[8], int l16) {
  const bool h3 = l16 & 8, h2 = l16 & 4, h1 = l16 & 2;
  float a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = (h3 ? x[4 + i] : x[i]) + dppf<0x128>(h3 ? x[i] : x[4 + i]);   // row_ror:8
#pragma unroll
  for (int i = 0; i < 2; ++i) b[i] = (h2 ? a[2 + i] : a[i]) + dppf<0x141>(h2 ? a[i] : a[2 + i]);   // row_half_mirror
  const float c = (h1 ? b[1] : b[0]) + dppf<0x4e>(h1 ? b[0] : b[1]);   // quad_perm [2,3,0,1]
  return c + dppf<0xb1>(c);                                           // quad_perm [1,0,3,2]
}

static_assert(std::is_standard_layout<AttnParams>::value, "kernarg offsets via offsetof");

template <int D, int RG, int PG, int TPW, int STAGES, bool SCORE>
__global__ __launch_bounds__(RG * PG * 64) void attn_split_kernel(const AttnParams p) {
  using C = Cfg<D, RG, PG, TPW, STAGES, SCORE>;
  constexpr int TN = C::TN;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int rg = wave / PG;   // row group: which row tiles
  const int pg = wave % PG;   // position group: which 32 positions of each KV tile
  const int l16 = lane & 15;
  const int kg = lane >> 4;
  // Workgroups go to the XCDs round-robin in dispatch order, so taking the KV
  // head from the low digits of the dispatch index keeps all splits of a head
  // on one XCD (with 8 KV heads: head g on XCD g); the combine blocks of that
  // head land there too and read its partials from that XCD's L2.
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int g = lin % p.Hkv;
  const int split = lin / p.Hkv;
  const int M = p.M;
  const int T = p.T;
  const int n_ctx = p.n_ctx;
  const int rows_total = n_ctx + T;
  const int ntiles_total = (rows_total + TN - 1) / TN;
  const int tiles_per_split = p.rows_per_split / TN;   // rows_per_split is a multiple of TN
  const int t_begin = split * tiles_per_split;
  const int t_end = min(t_begin + tiles_per_split, ntiles_total);
  const float c = p.scale_log2e;

  const uint16_t* __restrict__ kbase = p.k + (int64_t)g * p.s_head;
  const uint16_t* __restrict__ vbase = p.v + (int64_t)g * p.s_head;
  unsigned char* const qlds = lds + C::KV_BYTES;
  const unsigned int ring_off = lds_offset(lds);

  // ---- DMA staging of K and V tiles into ring slot tile % STAGES ----
  // Instruction j of a tensor covers ROWS_PER_DMA rows (j < DMA_PER_TENSOR),
  // issuing wave w (w < NI) taking j = w, w + NI, ... Lane l writes physical chunk
  // l % LANES_PER_ROW of its row; it fetches the logical chunk that the
  // swizzle maps there (K: chunk ^ row, V: chunk ^ 2*row, both mod NCH), which
  // keeps the later fragment reads conflict-free. The per-lane byte offsets
  // inside a tile are fixed, so they are computed once; a tile only moves the
  // buffer descriptor (scalar work). The descriptor ends at the last cache
  // row, so rows past it are never read.
  const int dma_row = lane / C::LANES_PER_ROW;
  const int dma_pc = lane % C::LANES_PER_ROW;
  const int64_t row_bytes = p.s_pos * 2;
  // When a wave's successive copies are NI * ROWS_PER_DMA rows apart and that
  // is a multiple of the swizzle period, the lane offsets repeat and only a
  // uniform row offset (the copy's scalar offset) changes: one VGPR per tensor.
  constexpr bool UNIFORM_STEP = (C::NI * C::ROWS_PER_DMA) % C::NCH == 0;
  constexpr int NOFF = UNIFORM_STEP ? 1 : C::DMA_T_PER_WAVE;
  unsigned int koff[NOFF], voff[NOFF];
#pragma unroll
  for (int jj = 0; jj < NOFF; ++jj) {
    const int r = (wave + jj * C::NI) * C::ROWS_PER_DMA + dma_row;
    koff[jj] = (unsigned int)(r * row_bytes) + ((dma_pc ^ (r & (C::NCH - 1))) << 4);
    voff[jj] = (unsigned int)(r * row_bytes) + ((dma_pc ^ ((2 * r) & (C::NCH - 1))) << 4);
  }
  const unsigned int jj_step = (unsigned int)(C::NI * C::ROWS_PER_DMA * row_bytes);
  auto issue = [&](int tile, bool is_v) {
    if (wave >= C::NI) return;
    const unsigned int slot = ring_off + (unsigned int)((tile % STAGES) * C::STAGE_BYTES + (is_v ? C::TILE_BYTES : 0));
    const int64_t tile_bytes = (int64_t)tile * TN * row_bytes;
    const int64_t rem = (int64_t)(rows_total - tile * TN) * row_bytes;
    const unsigned int nrec = rem > 0xffffffffll ? 0xffffffffu : (unsigned int)rem;
    const i32x4 desc = buffer_desc(reinterpret_cast<const unsigned char*>(is_v ? vbase : kbase) + tile_bytes, nrec);
#pragma unroll
    for (int jj = 0; jj < C::DMA_T_PER_WAVE; ++jj) {
      const int j = wave + jj * C::NI;
      if (C::DMA_PER_TENSOR % C::NI == 0 || j < C::DMA_PER_TENSOR)
        dma16_nt(desc, is_v ? voff[UNIFORM_STEP ? 0 : jj] : koff[UNIFORM_STEP ? 0 : jj],
                 UNIFORM_STEP ? jj * jj_step : 0u, slot + j * 1024);
    }
  };

  // ---- queries: B operand of S^T = K Q^T, from LDS ----
  // Row tiles: the nrt tiles of the KV head are shared evenly over the
  // gridDim.z blocks (at most RG * TPW each), and a block's R tiles go to its
  // row groups as evenly as possible (contiguous runs; the last R % RG
  // groups, whose waves issue no copies, take one tile more), so the SIMDs
  // carry nearly the same work: wave w runs on SIMD w % 4, and with PG = 2
  // row groups r and r + 2 share two SIMDs. The 1.5B shape's 9 row tiles go
  // 2 + 2 + 2 + 3 instead of 3 + 3 + 3 + 0, the 14B shape's 20 as two blocks
  // of 10 (2 + 2 + 3 + 3), not 12 + 8.
  const int nrt = (M + 15) / 16;
  const int per_blk = (nrt + (int)gridDim.z - 1) / (int)gridDim.z;
  const int rt_blk = blockIdx.z * per_blk;                  // first row tile of this block
  const int R = min(per_blk, nrt - rt_blk);                 // its live row tiles (<= RG * TPW)
  const int xr = RG - R % RG;                               // groups before the ones with a tile more
  const int nl = __builtin_amdgcn_readfirstlane(R / RG + (rg >= xr ? 1 : 0));   // this row group's
  const int lrt0 = rg * (R / RG) + max(0, rg - xr);         // its first tile within the block
  const int rt0 = rt_blk + lrt0;                            // its first row tile of the KV head
  // The block's query rows and the tree's ancestor words go to LDS by the
  // same asynchronous copy as K and V, before the K/V prologue: the first
  // tile's wait covers them, and no vector load is left pending into the loop
  // (the compiler would wait for such a load, and with it for every copy in
  // flight, before entering the loop). Queries are chunk-swizzled like K so
  // the B-fragment reads are conflict-free; rows past M are outside the
  // descriptor and are zeroed here instead (the copy skips them).
  unsigned char* const alds = qlds + C::Q_BYTES;
  // The first K tile is requested before the queries: the first tile's wait
  // counts only the copies issued after the queries, so it still covers them.
  if (t_begin < t_end) issue(t_begin, false);
  bool tile_on[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) tile_on[t] = t < nl;
  {
    // p is the kernel's only argument, so it starts the kernarg segment; its
    // ancestor words are read there (taking p's address would copy it to scratch)
    const unsigned char* kargs = (const unsigned char*)__builtin_amdgcn_kernarg_segment_ptr();
    if (wave == 0) {   // two words per node: one copy per 64 nodes
      const i32x4 adesc = buffer_desc(kargs + offsetof(AttnParams, anc), (unsigned int)(T * 16));
      dma16(adesc, (unsigned int)(lane * 16), ring_off + C::KV_BYTES + C::Q_BYTES);
      if (T > 64) dma16(adesc, (unsigned int)(1024 + lane * 16), ring_off + C::KV_BYTES + C::Q_BYTES + 1024);
    }
    constexpr int QD = C::ROWS_PER_BLOCK / C::ROWS_PER_DMA;   // copies of 1 KB
    const int q_rows = M - rt_blk * 16;
    for (int id = tid; id < C::ROWS_PER_BLOCK * C::NCH; id += C::NT)
      if (id / C::NCH >= q_rows) *reinterpret_cast<u32x4*>(qlds + id * 16) = u32x4{0u, 0u, 0u, 0u};
    const i32x4 qdesc = buffer_desc(p.q + ((int64_t)g * M + rt_blk * 16) * D, (unsigned int)(q_rows * C::ROWB));
#pragma unroll
    for (int jj = 0; jj < (QD + C::NI - 1) / C::NI; ++jj) {
      const int j = wave + jj * C::NI;
      const int r = j * C::ROWS_PER_DMA + dma_row;
      if (wave < C::NI && (QD % C::NI == 0 || j < QD))
        dma16(qdesc, (unsigned int)(r * C::ROWB + ((dma_pc ^ (r & (C::NCH - 1))) << 4)), ring_off + C::KV_BYTES + j * 1024);
    }
  }

  // O^T accumulators, plus one more tile per row tile that multiplies P by an
  // all-ones "value" fragment: every entry of it is the row's running sum of
  // the (f16-rounded) probabilities, so the sum needs no VALU adds or shuffles.
  f32x4 o[TPW][C::CT];
  f32x4 lsum[TPW];
  // m_thr is NEG_BIG until the first rescale and m_run + lazy_raw after it
  // (m_run is then above NEG_BIG); the score variant recomputes it from m_run
  // to free registers.
  const float lazy_raw = LAZY_LOG2 / c;   // slack in raw score units
  float m_run[TPW], m_thr[TPW];
  auto thr = [&](int t) { return SCORE ? (m_run[t] == NEG_BIG ? NEG_BIG : m_run[t] + lazy_raw) : m_thr[t]; };
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m_run[t] = NEG_BIG;
    m_thr[t] = NEG_BIG;
    lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) o[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (_Float16)1.0f;

  // ---- fused scores ----
  // After the reduce-scatter, lane (kg, l16) holds position
  // 16*b3 + 4*kg + 2*b2 + b1 of its wave's 32 (b = bits of l16). Row groups
  // past the first park their sums in LDS after a tile's second barrier; row
  // group 0 adds them after the next barrier (the next tile's first, or the
  // one after the loop) and stores; the slots are rewritten only after the
  // following second barrier.
  float* const sc_lds = reinterpret_cast<float*>(alds + C::ANC_BYTES);
  unsigned int* const vcnt = reinterpret_cast<unsigned int*>(alds + C::ANC_BYTES + C::SC_BYTES);
  const unsigned int cnt_lds = ring_off + (unsigned int)(C::KV_BYTES + C::Q_BYTES + C::ANC_BYTES + C::SC_BYTES);
  if constexpr (C::CNT_BYTES > 0)
    if (tid == 0) *vcnt = 0u;   // seen by every wave through the first tile's barrier
  float sig_keep = 0.f;
  auto score_slot = [&]() {
    const int l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return ((l & 8) << 1) + ((l >> 4) << 2) + ((l >> 1) & 3);
  };
  auto store_score = [&](int tl, float v) {
    const int pos = tl * TN + 32 * pg + score_slot();
    if ((l16 & 1) == 0 && pos < n_ctx) p.scores[(int64_t)g * n_ctx + pos] = v;
  };
  auto add_parked = [&](int tl) {
    if (tl * TN >= n_ctx) return;
    const int sq = score_slot();
    float v = sig_keep;
#pragma unroll
    for (int r = 1; r < RG; ++r) v += sc_lds[((r - 1) * PG + pg) * 32 + sq];
    store_score(tl, v);
  };

  // Ring schedule with two barriers per tile (the score variant). K of tile
  // i+STAGES is issued as soon as every wave has
  // finished S = K Q^T of tile i; V of tile i+STAGES-1 once every wave has
  // finished P V of tile i-1. Issue order per wave is therefore
  //   K(t0) V(t0) ... K(t0+S-2) V(t0+S-2) K(t0+S-1) | V(t0+S-1) K(t0+S) | V(t0+S) K(t0+S+1) | ...
  // K(i) is waited for before S of tile i, V(i) only before P V, so V(i)
  // lands while S is computed. Copies issued after K(i): at most S-1 K tiles
  // and S-1 V tiles (V(i) among them); after V(i): S-1 of each. An issuing
  // wave issues at least DMA_T_MIN copies per tensor tile, so waiting down to
  // that many per later tile lands the tile while the later copies stay in
  // flight. The other waves have no copies outstanding (their waits pass at
  // once) and see the tile through the barrier that follows each wait.
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (t_begin + st < t_end) {
      if (st > 0) issue(t_begin + st, false);   // K of the first tile went out first
      issue(t_begin + st, true);
    }
  // One barrier per tile (every eight-wave shape without score sums, whose
  // parked sums follow the two-barrier schedule): K and V of tile i+STAGES-1
  // go out together during tile i, once every wave is past the barrier of
  // tile i and so done with tile i-1 and its slot; no second barrier is
  // needed to refill a K slot (measured: T = 64 -2%, 14B -3%, 1.5B -4%). Each issuing wave converts
  // exactly the V rows its own copies wrote, after waiting for them, and the
  // other waves see the converted tile through the counter below. The
  // issuing waves request the next pair only after their share of the
  // conversion, so the counter is complete before the other waves need it
  // (14B -10%, 1.5B -4%, T = 64 -2%). With two row groups (each wave converts
  // its V fragments in registers) the issuing waves count their landed V
  // copies instead (T = 24 at 100K -1.7 us, at 8K -0.7 us); K of the next
  // tile goes out right after the barrier and V after the count (a further
  // -0.6 and -0.5 us; both after the count: K then had less than one tile's
  // lead; both at the barrier: +3 us).
  constexpr bool VCOUNT = !C::V_SHARED && !SCORE && C::NW >= 8;
  constexpr bool ONEBAR = (C::V_SHARED && !SCORE) || VCOUNT;
  if (!ONEBAR && t_begin + STAGES - 1 < t_end) issue(t_begin + STAGES - 1, false);

  constexpr int NK = C::DMA_T_MIN, VS = STAGES - 2;
  bf16x8 qreg[C::Q_REG ? TPW : 1][C::KSTEPS];
  // The tile loop computes NL row tiles per wave: TPW, or (four row groups)
  // TPW - 1 for the groups with fewer live tiles, so their SIMDs skip the
  // padded tiles' products and exponentials. Each is one straight loop with
  // no per-tile branches (tiles past a group's nl, if any, hold zero queries
  // or another group's rows; their results are never stored).
  auto tile_loop = [&](auto live) {
  constexpr int NL = decltype(live)::value;
  for (int tile = t_begin; tile < t_end; ++tile) {
    const int later = min(STAGES - 1, t_end - 1 - tile);   // tiles issued after this one
    if constexpr (ONEBAR) {
      // K(i): then V(i) and both tensors of min(S-2, later) later tiles
      if (later == 0) wait_vm<NK>();
      else if (later == 1 || VS < 2) wait_vm<(1 + 2 * (VS < 1 ? VS : 1)) * NK>();
      else wait_vm<(1 + 2 * (VS < 2 ? VS : 2)) * NK>();
      __builtin_amdgcn_s_barrier();  // K(tile) landed for every wave; tile-1 done everywhere
      if constexpr (VCOUNT)
        if (tile + STAGES - 1 < t_end) issue(tile + STAGES - 1, false);
    } else {
      // K(i): later K tiles, plus V(i) and min(S-2, later) more V tiles
      if (later == 0) wait_vm<NK>();
      else if (later == 1) wait_vm<(2 + (VS < 1 ? VS : 1)) * NK>();
      else if (later == 2) wait_vm<(3 + (VS < 2 ? VS : 2)) * NK>();
      else wait_vm<(4 + (VS < 3 ? VS : 3)) * NK>();
      __builtin_amdgcn_s_barrier();  // K(tile) landed for every wave; P V of tile-1 done everywhere
      if (tile + STAGES - 1 < t_end) issue(tile + STAGES - 1, true);
    }
    if constexpr (SCORE && RG > 1)
      if (rg == 0 && tile > t_begin) add_parked(tile - 1);

    const unsigned char* kl = lds + (tile % STAGES) * C::STAGE_BYTES;
    const unsigned char* vl = kl + C::TILE_BYTES;

    if constexpr (C::Q_REG) {
      if (tile == t_begin) {   // the queries have landed with the first K tile
#pragma unroll
        for (int t = 0; t < NL; ++t)
#pragma unroll
          for (int ks = 0; ks < C::KSTEPS; ++ks) {
            const int r = (lrt0 + t) * 16 + l16;
            qreg[t][ks] = *reinterpret_cast<const bf16x8*>(qlds + r * C::ROWB + (((4 * ks + kg) ^ (r & (C::NCH - 1))) << 4));
          }
      }
    }
    // ---- S^T = K Q^T over this wave's 32 positions ----
    f32x4 s[TPW][2];
#pragma unroll
    for (int t = 0; t < NL; ++t) s[t][0] = s[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      bf16x8 kf[2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const int row = 32 * pg + 16 * pt + l16;
        kf[pt] = *reinterpret_cast<const bf16x8*>(kl + row * C::ROWB + (((4 * ks + kg) ^ (row & (C::NCH - 1))) << 4));
      }
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        bf16x8 qv;
        if constexpr (C::Q_REG) {
          qv = qreg[t][ks];
        } else {
          const int r = (lrt0 + t) * 16 + l16;
          qv = *reinterpret_cast<const bf16x8*>(qlds + r * C::ROWB + (((4 * ks + kg) ^ (r & (C::NCH - 1))) << 4));
        }
        s[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], qv, s[t][0], 0, 0, 0);
        s[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1], qv, s[t][1], 0, 0, 0);
      }
    }
    if constexpr (!ONEBAR) {
      // V(tile): later tiles of both tensors may stay in flight. After the
      // barrier every wave's K reads of this tile are done: refill its K slot.
      if (later == 0) wait_vm<0>();
      else if (later == 1) wait_vm<2 * NK>();
      else if (later == 2) wait_vm<4 * NK>();
      else wait_vm<6 * NK>();
      __builtin_amdgcn_s_barrier();
      if (tile + STAGES < t_end) issue(tile + STAGES, false);
    }
    if constexpr (SCORE) {
      // this wave's share of sum_rows S for its 32 positions, after the
      // barrier so no wave waits for its S products before it
      if (tile * TN < n_ctx) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[j] = s[0][j >> 2][j & 3];
#pragma unroll
          for (int t = 1; t < NL; ++t) x[j] += s[t][j >> 2][j & 3];
        }
        const float sig = row16_scatter8(x, l16);
        if constexpr (RG == 1) store_score(tile, sig);
        else if (rg > 0 && (l16 & 1) == 0) sc_lds[((rg - 1) * PG + pg) * 32 + score_slot()] = sig;
        else sig_keep = sig;
      }
    }
    if ((tile + 1) * TN > rows_total) {
      // V rows past the cache were not loaded (the descriptor bounds the read)
      // and hold stale bits; P is exactly 0 there, but 0 * NaN would poison O.
      unsigned char* vw = lds + (tile % STAGES) * C::STAGE_BYTES + C::TILE_BYTES;
      for (int ch = tid; ch < C::TILE_BYTES / 16; ch += C::NT)
        if (tile * TN + ch / C::NCH >= rows_total) *reinterpret_cast<u32x4*>(vw + ch * 16) = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
    if constexpr (VCOUNT) {
      if (wave < C::NI) {   // this wave's V copies of the tile landed: count them, then V of the next tile
        // (K of the next tile went out at the barrier: it may be in flight, with the earlier pairs)
        if (later == 0) wait_vm<0>();
        else if (VS < 1) wait_vm<NK>();
        else if (later == 1) wait_vm<NK>();
        else wait_vm<3 * NK>();
        if (lane == 0) __hip_atomic_fetch_add(vcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (tile + STAGES - 1 < t_end) issue(tile + STAGES - 1, true);
      }
    }
    if constexpr (C::V_SHARED) {
      // V(tile) bf16 -> f16 in place, by the issuing waves only: the later
      // waves go on to their softmax meanwhile and wait for the count of
      // converted shares just before P V.
      if (wave < C::NI) {
        if constexpr (ONEBAR) {
          // V(i): both tensors of min(S-1, later) later tiles may stay in flight;
          // this wave converts exactly the rows its own copies wrote
          // (the next pair goes out after the conversion: only earlier pairs are in flight)
          if (later == 0 || VS < 1) wait_vm<0>();
          else wait_vm<2 * NK>();
        }
        unsigned char* vw = lds + (tile % STAGES) * C::STAGE_BYTES + C::TILE_BYTES;
        constexpr int NTI = C::NI * 64;
        constexpr int NCHK = C::TILE_BYTES / 16;
        constexpr int CPL = (NCHK + NTI - 1) / NTI;
        constexpr int BAT = CPL < 4 ? CPL : 4;   // chunks in registers at a time
        static_assert(CPL % BAT == 0, "conversion batches");
#pragma unroll
        for (int i0 = 0; i0 < CPL; i0 += BAT) {
          u32x4 w[BAT];
#pragma unroll
          for (int i = 0; i < BAT; ++i)
            if (NCHK % NTI == 0 || tid + (i0 + i) * NTI < NCHK) w[i] = *reinterpret_cast<const u32x4*>(vw + (tid + (i0 + i) * NTI) * 16);
#pragma unroll
          for (int i = 0; i < BAT; ++i)
            if (NCHK % NTI == 0 || tid + (i0 + i) * NTI < NCHK)
              *reinterpret_cast<u32x4*>(vw + (tid + (i0 + i) * NTI) * 16) =
                  u32x4{bf16x2_to_f16x2(w[i].x), bf16x2_to_f16x2(w[i].y), bf16x2_to_f16x2(w[i].z), bf16x2_to_f16x2(w[i].w)};
        }
        // this wave's share is written: count it (LDS operations of a wave complete in order)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(vcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if constexpr (ONEBAR)
          if (tile + STAGES - 1 < t_end) {
            issue(tile + STAGES - 1, false);
            issue(tile + STAGES - 1, true);
          }
      }
    }

    // the count of converted V shares (or landed V copies), read now and used
    // before P V (the read's latency passes during the softmax)
    unsigned int cnt_seen = 0u;
    if constexpr (C::V_SHARED || VCOUNT)
      cnt_seen = *(volatile LDS_AS unsigned int*)(LDS_AS unsigned char*)(unsigned char*)vcnt;
    // ---- tree mask and tail (only tiles reaching past the context) ----
    if ((tile + 1) * TN > n_ctx) {
      // a = offset into the tree rows; visible iff a committed row (a < 0)
      // or an ancestor-or-self tree node. Branch-free selects.
      const int a0 = tile * TN + 32 * pg + 4 * kg - n_ctx;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int row = (rt0 + t) * 16 + l16;
        // bit j of win = tree node a0 + j visible to this row (two words per
        // node: nodes 0-63, 64-127); the lane's positions lie in [a0, a0 + 20)
        const int node = row < M ? row % T : 0;
        const unsigned __int128 m = (unsigned __int128)reinterpret_cast<const uint64_t*>(alds)[2 * node] |
                                    ((unsigned __int128)reinterpret_cast<const uint64_t*>(alds)[2 * node + 1] << 64);
        const unsigned int win = a0 >= 0 ? (a0 < 128 ? (unsigned int)(m >> a0) : 0u)
                                         : (-a0 < 32 ? (unsigned int)(m << -a0) : 0u);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int a = a0 + 16 * pt + i;
            const unsigned int bit = (win >> (16 * pt + i)) & 1u;
            const unsigned int vis = (unsigned int)(a < 0) | ((unsigned int)(a < T) & bit);
            s[t][pt][i] = vis ? s[t][pt][i] : -INFINITY;
          }
      }
    }

    // ---- online softmax, P -> f16 B fragments ----
    // Row tiles past M hold zero queries and are computed like the others (their
    // results are never stored), so the tile body has no per-tile branches and
    // the scheduler can overlap one tile's exponentials with another's MFMAs.
    // A row's four lanes hold the same threshold, so whether any row must
    // rescale follows from each lane's own maximum: the row maximum across
    // the four lanes is formed only on the rare tiles that rescale.
    float mx[TPW];
    bool bump_any = false;
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      mx[t] = lane_max8(s[t][0], s[t][1]);
      bump_any |= mx[t] > thr(t);
    }
    // Lazy rescale: the reference max only moves when the tile max exceeds it
    // by more than 2^8 in probability, so p = exp2(s*c - m*c) stays <= 256
    // (exact enough in f16) and the O rescale is rare.
    if (__ballot(bump_any)) {
#pragma unroll
      for (int t = 0; t < NL; ++t) mx[t] = group4_max(mx[t]);
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const bool bump = mx[t] > thr(t);
        const float m_new = bump ? mx[t] : m_run[t];
        const float alpha = __builtin_amdgcn_exp2f((m_run[t] - m_new) * c);
        m_run[t] = m_new;
        m_thr[t] = bump ? m_new + lazy_raw : m_thr[t];
        lsum[t] *= alpha;
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) o[t][ct] *= alpha;
      }
    }
    f16x8 pfrag[TPW];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const float nmc = -m_run[t] * c;
      f16x8 f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[t][0][i], c, nmc));
        f[4 + i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[t][1][i], c, nmc));
      }
      pfrag[t] = f;
      lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, f, lsum[t], 0, 0, 0);
    }

    if constexpr (C::V_SHARED || VCOUNT) {
      // Wait until every issuing wave has counted its share of this tile's
      // conversion (or its landed V copies), instead of a barrier: the
      // issuing waves go on to P V while the later waves still run their
      // softmax. Bounded (the counts come early in the tile, long before any
      // wave gets here), so a wave never waits without end.
      const unsigned int want = (unsigned int)(C::NI * (tile - t_begin + 1));
      // (the count read before the softmax is normally complete already)
      for (int spin = 0; spin < (1 << 16) && __builtin_amdgcn_readfirstlane(cnt_seen) < want; ++spin) {
        unsigned int v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(cnt_lds) : "memory");
        if (__builtin_amdgcn_readfirstlane(v) >= want) break;
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");
    }
    // ---- O^T += V^T P^T (V^T fragments by LDS transpose reads, f16 from the shared
    //      conversion or bf16 -> f16 in registers) ----
    {
      const int r_lo = 32 * pg + 4 * kg + (l16 >> 2);
      const int swz = (2 * r_lo) & (C::NCH - 1);  // same for r_lo + 16
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
        const int chunk = 2 * ct + ((l16 & 3) >> 1);
        const int off = ((chunk ^ swz) << 4) + ((l16 & 1) << 3);
        const LDS_AS s16x4* a_lo = (const LDS_AS s16x4*)(const LDS_AS unsigned char*)(vl + r_lo * C::ROWB + off);
        const LDS_AS s16x4* a_hi = (const LDS_AS s16x4*)(const LDS_AS unsigned char*)(vl + (r_lo + 16) * C::ROWB + off);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)a_lo);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)a_hi);
        const u32x4 wb = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        f16x8 vf;
        if constexpr (C::V_SHARED)
          vf = __builtin_bit_cast(f16x8, wb);
        else
          vf = __builtin_bit_cast(
              f16x8, u32x4{bf16x2_to_f16x2(wb.x), bf16x2_to_f16x2(wb.y), bf16x2_to_f16x2(wb.z), bf16x2_to_f16x2(wb.w)});
#pragma unroll
        for (int t = 0; t < NL; ++t)
          o[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pfrag[t], o[t][ct], 0, 0, 0);
      }
    }
  }

  };
  if constexpr (RG >= 4 && TPW >= 2) {
    if (nl >= TPW) tile_loop(std::integral_constant<int, TPW>{});
    else tile_loop(std::integral_constant<int, TPW - 1>{});
  } else {
    tile_loop(std::integral_constant<int, TPW>{});
  }

  if constexpr (SCORE && RG > 1) {
    bar();   // the last tile's parked sums
    if (rg == 0 && t_end > t_begin) add_parked(t_end - 1);
  }

  // ---- per-row probability sums (every entry of lsum holds the full sum) ----
  float l_run[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) l_run[t] = lsum[t][0];

  // ---- merge the PG position groups of each row group, then store ----
  // Wave (rg, pg) merges and stores channel tiles pg, pg + PG, ... of its row
  // group: it keeps those in registers and parks the other channel tiles and
  // its (m, l) in LDS, MERGE_RT row tiles per round (all of LDS is free after
  // the loop). Output: normalised rows (single split) or the split's partial
  // (O^T, m, l).
  constexpr int CTW = C::CT / PG;   // channel tiles merged and stored per wave
  // The score variant derives the store addresses from a lane id the compiler
  // cannot move above the loop: hoisted there, they would be kept in (short)
  // registers through the whole loop.
  int lane_st = lane;
  if constexpr (SCORE) asm volatile("" : "+v"(lane_st));
  const int l16_st = lane_st & 15, kg_st = lane_st >> 4;
  auto store = [&](int t, float mu, float wsum, const f32x4 (&om)[CTW]) {
    const int row = (rt0 + t) * 16 + (SCORE ? l16_st : l16);
    const int kgs = SCORE ? kg_st : kg;
    if (!tile_on[t] || row >= M) return;
    if (p.n_split == 1) {
      const float inv = 1.0f / wsum;
      float* dst = p.out + ((int64_t)g * M + row) * D + 4 * kgs;
#pragma unroll
      for (int i = 0; i < CTW; ++i) *reinterpret_cast<f32x4*>(dst + (pg + i * PG) * 16) = om[i] * inv;
    } else {
      // a split can see none of a row's positions (tree rows past its start
      // that are not the row's ancestors): sum 0, weight 0 in the merge
      const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
      const int64_t prow = ((int64_t)split * p.Hkv + g) * M + row;
      uint16_t* dst = p.part_acc + prow * D + 4 * kgs;
#pragma unroll
      for (int i = 0; i < CTW; ++i) {
        const f32x4 x = om[i] * inv;
        const f16x4 h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
        *reinterpret_cast<f16x4*>(dst + (pg + i * PG) * 16) = h;
      }
      if (pg == 0 && kgs == 0) {
        p.part_ml[prow * 2 + 0] = mu;
        p.part_ml[prow * 2 + 1] = wsum;
      }
    }
  };
  if constexpr (PG == 1) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      f32x4 om[CTW];
#pragma unroll
      for (int i = 0; i < CTW; ++i) om[i] = o[t][i];
      store(t, m_run[t], l_run[t], om);
    }
  } else {
    constexpr int RT = C::MERGE_RT;
    constexpr int OFF_ML = 64 * C::CT_OUT * 16;   // m and l after the parked O^T fragments in a slot
#pragma unroll
    for (int t0 = 0; t0 < TPW; t0 += RT) {
      // LDS-only barriers: the partial stores of the previous round may stay
      // in flight (__syncthreads would wait for them).
      bar();  // the ring (or the previous round) is free
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        const int t = t0 + u;
        if (t >= TPW) break;
        unsigned char* my = lds + ((u * RG + rg) * PG + pg) * C::MSLOT;
        // channel tiles of the other waves' share, in ascending order
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
          if (ct % PG != pg) {
            const int pos = (ct / PG) * (PG - 1) + ct % PG - (ct % PG > pg ? 1 : 0);
            *reinterpret_cast<f32x4*>(my + (pos * 64 + lane) * 16) = o[t][ct];
          }
        if (kg == 0) {
          reinterpret_cast<float*>(my + OFF_ML)[l16] = m_run[t];
          reinterpret_cast<float*>(my + OFF_ML)[16 + l16] = l_run[t];
        }
      }
      bar();
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        const int t = t0 + u;
        if (t >= TPW) break;
        const unsigned char* grp = lds + (u * RG + rg) * PG * C::MSLOT;
        float mq[PG], wq[PG];
        float mu = NEG_BIG;
#pragma unroll
        for (int q = 0; q < PG; ++q) {
          mq[q] = q == pg ? m_run[t] : reinterpret_cast<const float*>(grp + q * C::MSLOT + OFF_ML)[l16];
          mu = fmaxf(mu, mq[q]);
        }
        float wsum = 0.f;
#pragma unroll
        for (int q = 0; q < PG; ++q) {
          wq[q] = __builtin_amdgcn_exp2f((mq[q] - mu) * c);
          wsum += wq[q] * (q == pg ? l_run[t] : reinterpret_cast<const float*>(grp + q * C::MSLOT + OFF_ML)[16 + l16]);
        }
        f32x4 om[CTW];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
          if (ct % PG == pg) {
            // in wave q's slot this channel tile sits after (ct / PG) * (PG - 1)
            // tiles of earlier groups and the tiles pg' < pg, pg' != q, of its own group
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < PG; ++q) {
              if (q == pg) {
                acc += wq[q] * o[t][ct];
              } else {
                const int pos = (ct / PG) * (PG - 1) + pg - (q < pg ? 1 : 0);
                acc += wq[q] * *reinterpret_cast<const f32x4*>(grp + q * C::MSLOT + (pos * 64 + lane) * 16);
              }
            }
            om[ct / PG] = acc;
          }
        store(t, mu, wsum, om);
      }
    }
  }
}

// Log-sum-exp merge of the split partials: one wave per output row, no LDS.
// Lane (sg, cg) holds the CPL = d/16 channels of group cg (one 16- or 8-byte
// f16 load per split) of the splits sg, sg + 4, ... (four split groups per
// wave), merges them in one online pass with U splits' loads in flight, then
// the split groups merge across lanes with the gfx950 row / half swaps, in a
// fixed order (bitwise repeatable). A split's weight is l_s * 2^((m_s - m) c)
// and its normalised output enters with that weight.
template <int D, int U>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnParams p) {
  constexpr int CPL = D / 16;               // channels per lane
  constexpr int CG = D / CPL;               // channel groups per row (16)
  constexpr int SG = 64 / CG;               // split groups per wave (4)
  // U: splits in flight per lane
  static_assert(SG == 4, "one row per wave");
  typedef _Float16 hv __attribute__((ext_vector_type(CPL)));
  const int lane = threadIdx.x & 63;
  const int nrows = p.Hkv * p.M;
  // block b: KV head b % Hkv (the split kernel placed that head's splits on
  // the XCD this block lands on), rows 4 * (b / Hkv) .. + 3 of the head
  const int gh = blockIdx.x % p.Hkv;
  const int r = (blockIdx.x / p.Hkv) * 4 + (int)(threadIdx.x >> 6);
  if (r >= p.M) return;   // wave-uniform
  const int row = gh * p.M + r;   // g * M + r
  const int sg = lane / CG, cg = lane % CG;
  const float c = p.scale_log2e;
  const int64_t sstride = nrows;

  // Partial maxima are finite (running maxima start at a finite floor); -inf
  // marks "no split here" and gets weight 0.
  float m_loc = -INFINITY, l_loc = 0.f;
  float a_loc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) a_loc[j] = 0.f;
  for (int s0 = sg; s0 < p.n_split; s0 += SG * U) {
    float mv[U], lv[U];
    hv av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SG;
      const bool in = s < p.n_split;
      const int64_t pr = (int64_t)(in ? s : s0) * sstride + row;
      const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + pr * 2);
      mv[u] = in ? ml.x : -INFINITY;
      lv[u] = in ? ml.y : 0.f;
      av[u] = *reinterpret_cast<const hv*>(p.part_acc + pr * D + CPL * cg);
    }
    float mn = m_loc;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, mv[u]);
    const float sc = __builtin_amdgcn_exp2f((m_loc - mn) * c);   // 0 on the first round
    l_loc *= sc;
#pragma unroll
    for (int j = 0; j < CPL; ++j) a_loc[j] *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __builtin_amdgcn_exp2f((mv[u] - mn) * c) * lv[u];
      l_loc += w;
#pragma unroll
      for (int j = 0; j < CPL; ++j) a_loc[j] += w * (float)av[u][j];
    }
    m_loc = mn;
  }
  // merge the split groups: lanes l and l ^ 16, then l and l ^ 32
  auto merge = [&](auto swap) {
    const auto mm = swap(__float_as_uint(m_loc));
    const float m0 = __uint_as_float(mm[0]), m1 = __uint_as_float(mm[1]);
    const float mu = fmaxf(m0, m1);
    // the pair (lower group, upper group) in the same order in both lanes
    const float w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - mu) * c);
    const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - mu) * c);
    const auto ll = swap(__float_as_uint(l_loc));
    l_loc = w0 * __uint_as_float(ll[0]) + w1 * __uint_as_float(ll[1]);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const auto aa = swap(__float_as_uint(a_loc[j]));
      a_loc[j] = w0 * __uint_as_float(aa[0]) + w1 * __uint_as_float(aa[1]);
    }
    m_loc = mu;
  };
  merge([](unsigned int x) { return __builtin_amdgcn_permlane16_swap(x, x, false, false); });
  merge([](unsigned int x) { return __builtin_amdgcn_permlane32_swap(x, x, false, false); });
  if (sg == 0) {
    const float inv = 1.0f / l_loc;
    float* dst = p.out + (int64_t)row * D + CPL * cg;
#pragma unroll
    for (int j = 0; j < CPL; j += 4)
      *reinterpret_cast<f32x4*>(dst + j) = f32x4{a_loc[j], a_loc[j + 1], a_loc[j + 2], a_loc[j + 3]} * inv;
  }
}

struct KernelChoice {
  int rg, pg, tpw;
};


// Row tiles per KV head -> (row groups, position groups, row tiles per wave).
// From 4 row tiles on the workgroup has 8 waves (two per SIMD); every choice
// keeps the accumulators in registers without spilling. Past 16 row tiles
// the rows go to several workgroups (grid.z) of 12 or 16 row tiles, whichever
// pads fewer. Measured at 100K: T = 48 (12 row tiles) 132 us with (4, 2, 3)
// against 164 us with four waves (4, 1, 3); T = 64 (16) 154 against 185 us
// with (4, 1, 4); 14B T = 64 (20) 214 against 240 us with (4, 1, 5); the
// 1.5B shape (9 row tiles) 46.1 us with (4, 2, 3) (three padded row tiles,
// eight waves) against 48.0 us with six waves (3, 2, 3), whose SIMDs hold
// two waves or one.
KernelChoice choose(int nrt) {
  if (nrt <= 1) return {1, 4, 1};
  if (nrt == 2) return {1, 4, 2};
  if (nrt == 3) return {1, 4, 3};
  if (nrt == 4) return {2, 4, 2};
  if (nrt <= 6) return {2, 4, 3};
  if (nrt <= 8) return {4, 2, 2};
  if (nrt <= 12) return {4, 2, 3};
  if (nrt <= 16) return {4, 2, 4};
  const int pad3 = (nrt + 11) / 12 * 12, pad4 = (nrt + 15) / 16 * 16;
  return pad3 < pad4 ? KernelChoice{4, 2, 3} : KernelChoice{4, 2, 4};
}

// K/V ring depth: three tiles (two in flight while one is computed), or two
// when three would not fit in the 160 KB of LDS next to the queries.
template <int D, int RG, int PG, int TPW>
hipError_t launch_split(const AttnParams& p, int nz, hipStream_t stream) {
  constexpr int STAGES = Cfg<D, RG, PG, TPW, 3>::LDS_BYTES <= 160 * 1024 ? 3 : 2;
  static_assert(Cfg<D, RG, PG, TPW, STAGES, true>::LDS_BYTES <= 160 * 1024, "LDS budget");
  dim3 grid(p.n_split, p.Hkv, nz);
  if (p.scores)
    hipLaunchKernelGGL((attn_split_kernel<D, RG, PG, TPW, STAGES, true>), grid, dim3(RG * PG * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, RG, PG, TPW, STAGES, false>), grid, dim3(RG * PG * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const AttnParams& p, const KernelChoice& kc, int nz, hipStream_t stream) {
#define TS_CASE(RG_, PG_, TPW_) \
  if (kc.rg == RG_ && kc.pg == PG_ && kc.tpw == TPW_) return launch_split<D, RG_, PG_, TPW_>(p, nz, stream);
  TS_CASE(1, 4, 1)
  TS_CASE(1, 4, 2)
  TS_CASE(1, 4, 3)
  TS_CASE(2, 4, 2)
  TS_CASE(2, 4, 3)
  TS_CASE(4, 2, 2)
  TS_CASE(4, 2, 3)
  TS_CASE(4, 2, 4)
#undef TS_CASE
  return hipErrorInvalidValue;
}

int row_blocks_for(int M) {
  const int nrt = (M + 15) / 16;
  const KernelChoice kc = choose(nrt);
  const int per = kc.rg * kc.tpw;
  return (nrt + per - 1) / per;
}

// Split granularity in positions: the K/V tile of the form the rows take
// (32 positions per position group), so a split ends on a tile boundary and
// the splits can be spread over every compute unit (the 1.5B shape, 64-position
// tiles: 121 splits of 13 tiles per KV head instead of 112 of 14).
int split_tile(int M) {
  const KernelChoice kc = choose((M + 15) / 16);
  return 32 * kc.pg;
}

}  // namespace

int attn_row_blocks(int32_t T, int32_t Hq, int32_t Hkv) { return row_blocks_for((Hq / Hkv) * T); }

int attn_auto_split(int32_t rows_total, int32_t T, int32_t Hq, int32_t Hkv, int32_t d) {
  (void)d;
  const int M = (Hq / Hkv) * T;
  const int tn = split_tile(M);
  const int ntiles = (rows_total + tn - 1) / tn;
  const int nz = row_blocks_for(M);
  const int target_wg = 256;  // one resident workgroup on each of 256 compute units
  int s = (target_wg + Hkv * nz - 1) / (Hkv * nz);
  if (s > ntiles) s = ntiles;
  if (s < 1) s = 1;
  return s;
}

void attn_split_plan(int32_t rows_total, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                     int32_t n_split_req, int32_t* n_split_eff, int32_t* rows_per_split) {
  const int tn = split_tile((Hq / Hkv) * T);
  const int ntiles = (rows_total + tn - 1) / tn;
  int s = n_split_req > 0 ? n_split_req : attn_auto_split(rows_total, T, Hq, Hkv, d);
  if (s > ntiles) s = ntiles;
  if (s < 1) s = 1;
  const int tps = (ntiles + s - 1) / s;
  *rows_per_split = tps * tn;
  *n_split_eff = (ntiles + tps - 1) / tps;
}

size_t attn_workspace_bytes(int32_t rows_total, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                            int32_t n_split_req) {
  int32_t s, tps;
  attn_split_plan(rows_total, T, Hq, Hkv, d, n_split_req, &s, &tps);
  if (s <= 1) return 0;
  const size_t M = (size_t)(Hq / Hkv) * T;
  return (size_t)s * Hkv * M * ((size_t)d * 2 + 2 * sizeof(float));   // f16 outputs, then (m, l) pairs
}

hipError_t launch_attention(const AttnParams& p, hipStream_t stream) {
  const int nrt = (p.M + 15) / 16;
  const KernelChoice kc = choose(nrt);
  const int nz = row_blocks_for(p.M);
  if (p.scores && nz != 1) return hipErrorInvalidValue;   // the host checks this first
  hipError_t e = p.d == 128 ? launch_split_d<128>(p, kc, nz, stream) : launch_split_d<64>(p, kc, nz, stream);
  if (e != hipSuccess || p.n_split == 1) return e;
  const dim3 cgrid(p.Hkv * ((p.M + 3) / 4));   // one row per wave, four waves per block
  // eight splits in flight per lane cover 32 splits in one round; more splits
  // (few KV heads: 112 at the 1.5B shape) take all of a lane's loads at once
  if (p.n_split <= 32) {
    if (p.d == 128)
      hipLaunchKernelGGL((attn_combine_kernel<128, 8>), cgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_combine_kernel<64, 8>), cgrid, dim3(256), 0, stream, p);
  } else {
    if (p.d == 128)
      hipLaunchKernelGGL((attn_combine_kernel<128, 32>), cgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_combine_kernel<64, 32>), cgrid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ts
