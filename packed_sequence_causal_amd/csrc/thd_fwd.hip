// Forward kernel: causal + EOD-reset attention for one rank's query tiles
// against rank-major gathered K/V (gfx950, bf16 MFMA, fp32 accumulate).
//
// The operation is the one of "kvallgather cp thd load balance" (Ascend/
// MindSpeed, "What this PR does / why we need it?": THD attention with direct
// rank-major K/V indexing in a single fused call; "Does this PR introduce any
// user-facing change?": causal attention with the mask reset at every EOD).
//
// Work decomposition. One workgroup (4 waves, 256 lanes) handles one work
// item (a query tile, or a part of its key range when the planner splits the
// longest tiles for balance) of one kv head: block_t tokens x G q heads = up to 128 rows, token-major
// (row = token * G + head-in-group), 32 rows per wave. All G heads of a kv head
// share every K/V tile, so a K/V tile loaded once into LDS feeds 128 rows even
// when tiles hold few tokens. Workgroup b takes kv head b % Hkv and work item
// b / Hkv: items are dispatched longest first, and since workgroups are
// spread round robin over the 8 XCDs, with Hkv = 8 each XCD (and its L2) serves
// a single kv head.
//
// Per KV tile of 64 keys (only the tiles from the document start up to the
// tile's last row are visited):
//   * K and V rows are gathered straight from HBM into a two-stage LDS ring
//     with global_load_lds_dwordx4 (16 bytes per lane, no register staging):
//     the next tile streams in while the current one is computed. The row of
//     each key comes from the gathered-row map (no reorder copy of K/V); those
//     indices are fetched one tile further ahead. Rows are stored with their
//     16-byte chunks XOR-swizzled by row so that the MFMA operand reads below
//     hit distinct LDS banks;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T from
//     registers): each lane then holds one query row (lane % 32) and 16 keys
//     per 32-key block, so row reductions are in-lane plus one exchange with
//     lane ^ 32;
//   * the causal compare runs only on tiles past the first row's position;
//   * online softmax in the log2 domain (scale * log2(e) folded into one FMA,
//     v_exp_f32); a row's running maximum is only raised when its maximum
//     grows by more than 8 (2^8 headroom in fp32 and bf16), which skips most
//     rescales of the accumulator and is exact up to rounding;
//   * O^T += V^T P^T: the S^T register layout is already the B-operand layout
//     of P^T, so P never leaves registers; the V^T operand is read from the
//     row-major V tile with ds_read_b64_tr_b16, which hands each lane of a
//     16-lane group one column of the 4 x 16 block formed by the group's four
//     8-byte row pieces (4 consecutive keys of one V column).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <mutex>
#include <vector>

#include "internal.h"

namespace thd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Four waves of 64 lanes per workgroup, one 32-row block each, two workgroups
// per CU: two waves share each SIMD and hide each other's latencies. (Two
// blocks per wave at one wave per SIMD halves LDS reads per MFMA but measured
// 1.6x slower: the latency hiding between waves matters more.)
constexpr int kRowBlocks = 1;
constexpr int kFwdWaves = kRowsPerWg / (32 * kRowBlocks);
constexpr int kFwdThreads = kFwdWaves * 64;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;
constexpr int kWaitVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;    // s_waitcnt lgkmcnt(0)
template <int N>
constexpr int kWaitLgkmKB = 0xC07F | (N << 8);   // s_waitcnt lgkmcnt(N)

// 16-byte global -> LDS copy: lane i's 16 bytes land at lds + 16 * i (lds is
// wave-uniform). Kept as a function taking a named pointer: handing the
// builtin a pointer expression directly inside a kernel template makes the
// host pass drop that kernel's launch stub.
__device__ __forceinline__ void load_lds16(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
}

// Splits (x0, x1) into two packed bf16 pairs: hi holds x truncated to bf16
// (the upper half of each float, one byte permute), lo holds x - hi (exact in
// fp32) rounded to bf16. hi + lo equals x to within 2^-16 of |x|.
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
  const unsigned u0 = __builtin_bit_cast(unsigned, x0), u1 = __builtin_bit_cast(unsigned, x1);
  hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
  const float r0 = x0 - __builtin_bit_cast(float, u0 & 0xffff0000u);
  const float r1 = x1 - __builtin_bit_cast(float, u1 & 0xffff0000u);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

// Position of 16-byte chunk c of LDS row r: c ^ swz(r). The XOR stays inside
// an aligned group of 8 (or 16) chunks, so it never leaves the row.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (r >> 1) & 7;
  }
}

template <int DQK, int DV, int BN_>
struct FwdShape {
  static constexpr int BN = BN_;
  static constexpr int KCPR = DQK / 8;            // 16-byte chunks per K row
  static constexpr int VCPR = DV / 8;
  static constexpr int KROWB = DQK * 2;
  static constexpr int VROWB = DV * 2;
  static constexpr int KBYTES = BN * KROWB;       // one K tile in LDS
  static constexpr int VBYTES = BN * VROWB;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int K_IPW = BN * KCPR / 64 / kFwdWaves;   // 1 KB loads per wave per tile
  static constexpr int V_IPW = BN * VCPR / 64 / kFwdWaves;
  static constexpr bool SAME_ROWS = (KCPR == VCPR);
  static constexpr int NROWS = SAME_ROWS ? K_IPW : K_IPW + V_IPW;  // row indices per lane per tile
  static constexpr int KSTEPS = DQK / 16;
  static constexpr int DVB = DV / 32;
  static constexpr int KB = BN / 32;        // 32-key blocks per KV tile (S^T accumulators)
  static constexpr int TS = BN / 16;        // 16-key steps of the PV product
  static_assert(BN % 32 == 0, "KV tiles hold whole 32-key blocks");
  static_assert(BN * KCPR % (64 * kFwdWaves) == 0 && BN * VCPR % (64 * kFwdWaves) == 0,
                "tiles must split into whole 1 KB loads per wave");
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims must suit the MFMA tiles");
  static_assert(KCPR == 8 || KCPR == 16 || KCPR == 24, "chunk swizzle needs 8, 16 or 24 chunks");
  static_assert(VCPR == 8 || VCPR == 16, "V chunk swizzle needs 8 or 16 chunks");
};

// EXACT: P enters the PV product as a bf16 (hi, lo) pair and O is also written
// in fp32 (p.o_f32): O is then exact up to fp32 accumulation, so the backward
// can take D = rowsum(dO * O) from it.
// Workgroups per CU: two with 64-key tiles (64 KB of LDS ring each), three
// with 32-key tiles (the register budget then drops to 168 per lane).
template <int BN>
constexpr int kFwdOccupancy = BN == kBlockNShort ? 3 : 2;

// RANGED: one forward pass of a pass plan (all-gather overlap): a workgroup
// takes one tile (p.pass_order) and walks each of the tile's runs (absolute
// key ranges [first key, end key), p.pass_runs) in turn with the same online
// softmax, then merges its result straight into the caller's running state.
// PACKED: a packed plan's items, some of whose tiles are packed tiles (rows of
// several documents; short-segment packing): such a tile's rows, their key
// windows and its key slots come from pack_rows / pack_keys, every KV tile
// takes the two-sided window compare, and a wave skips the KV tiles its rows'
// windows do not reach.
template <int DQK, int DV, bool EXACT, int BN_, bool RANGED = false, bool PACKED = false>
__global__ __launch_bounds__(kFwdThreads, kFwdOccupancy<BN_>) void thd_fwd_kernel(FwdParams p) {
  using S = FwdShape<DQK, DV, BN_>;
  constexpr int BN = S::BN;
  constexpr int RB = kRowBlocks;
  // The two ring stages are separate arrays, and the tile loop is unrolled by
  // two so that each step names its stages statically: the compiler can then
  // tell that the transpose reads of one stage do not alias the in-flight LDS
  // writes into the other, and does not wait for the next tile's loads before
  // reading the current one.
  __shared__ __attribute__((aligned(1024))) char smem0[S::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[S::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int half = lane >> 5;        // which 32-lane half (recomputed for the epilogue)
  int lrow = lane & 31;

  // Work item: KV tiles [kv_begin, kv_end) of one query tile (a whole tile
  // unless its key range is split), for kv head blockIdx.x % Hkv. A pass
  // (RANGED) takes a whole tile and its n_runs runs of this pass's keys.
  const int kvh = blockIdx.x % p.hkv;
  int tile, kv_begin, kv_end, part, n_runs = 1;
  const int32_t* item;
  const int32_t* runs = nullptr;
  if constexpr (RANGED) {
    const int32_t* sp = p.splits + size_t(p.pass_order[blockIdx.x / p.hkv]) * 4;
    tile = sp[0];
    n_runs = sp[2];
    runs = p.pass_runs + size_t(sp[1]) * 8;
    item = runs;
    kv_begin = 0;
    kv_end = n_runs > 0 ? runs[4] : 0;
    part = -1;
  } else {
    item = p.items + size_t(blockIdx.x / p.hkv) * 4;
    tile = item[0];
    kv_begin = item[1];
    kv_end = item[2];
    part = item[3];
  }
  const int32_t* td = p.tiles + size_t(tile) * 8;
  // A packed tile's td[1] is its first row in pack_rows and td[5] its first
  // key slot; its slots are numbered from 0 and fill td[6] whole KV tiles.
  const bool packed_tile = PACKED && td[0] < 0;
  const int q_local0 = td[0];
  const int q_glob0 = td[1];
  const int n_rows = td[2];
  // KV tiles start at the document's first key (a pass plan's item: at its
  // run's first key); keys from key_hi on are seen by no row of the item.
  int kv_start = RANGED ? (n_runs > 0 ? item[1] : 0) : (packed_tile ? 0 : td[5]);
  int n_full = RANGED ? (n_runs > 0 ? item[5] : 0) : td[7];
  int key_hi = RANGED ? (n_runs > 0 ? item[2] : 1) : (packed_tile ? td[6] * BN : q_glob0 + n_rows);
  // Rows at or past the document's last real token are padding: written as
  // O = 0, LSE = +inf (tokens are in position order within a plain tile; a
  // packed row carries its own flag).
  const int n_real = packed_tile ? 0 : min(max(p.doc_end[td[3]] - q_glob0, 0), n_rows);
  int key_last = key_hi - 1;

  // Row block rb of this wave holds rows 32 * (RB * wave + rb) + lane % 32.
  const int G = p.group;
  // qpos: the last key (slot) a row sees. Packed plans only: qlo, the first;
  // for rows of a packed tile, pk_row and pk_real hold its local query row
  // and whether it is real (other kernels derive both from the token when
  // they store, which keeps them out of registers during the tile loop).
  int tok[RB], head[RB], qpos[RB], qlo[RB], pk_row[RB];
  bool valid[RB], rb_active[RB], pk_real[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row0 = 32 * (RB * wave + rb);
    const int row = row0 + lrow;
    tok[rb] = row / G;
    head[rb] = kvh * G + (row - tok[rb] * G);
    valid[rb] = tok[rb] < n_rows;
    // The causal compare also ends a pass item's range at key_hi.
    qpos[rb] = valid[rb] ? (RANGED ? min(q_glob0 + tok[rb], key_last) : q_glob0 + tok[rb]) : INT_MAX;
    qlo[rb] = 0;
    pk_row[rb] = q_local0 + tok[rb];
    pk_real[rb] = tok[rb] < n_real;
    if constexpr (PACKED) {
      if (packed_tile) {
        const i32x4 pr = valid[rb] ? *reinterpret_cast<const i32x4*>(p.pack_rows + 4 * size_t(q_glob0 + tok[rb]))
                                   : i32x4{0, 0, INT_MAX, 0};
        pk_row[rb] = pr[0];
        qlo[rb] = pr[1];
        qpos[rb] = pr[2];
        pk_real[rb] = pr[3] != 0;
      }
    }
    rb_active[rb] = row0 / G < n_rows;          // wave-uniform
  }
  const bool wave_active = rb_active[0];

  const __bf16* __restrict__ qp = static_cast<const __bf16*>(p.q);
  const char* __restrict__ kb = static_cast<const char*>(p.k);
  const char* __restrict__ vb = static_cast<const char*>(p.v);
  const int32_t* __restrict__ kv_row = packed_tile ? p.pack_keys + td[5] : p.kv_row;
  const int hkv = p.hkv;

  // Q^T operand: lane holds Q[row][16*st + 8*half .. +7] for each k-step.
  // A packed tile's rows are known only once pack_rows has arrived, so its Q
  // loads go out after the first KV tile's copies (its key rows are fetched
  // alongside pack_rows): the first tile then waits on one dependent load,
  // as in a plain tile, instead of two.
  bf16x8 qf[RB][S::KSTEPS];
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qrow = PACKED ? pk_row[rb] : q_local0 + tok[rb];
      const __bf16* qsrc = qp + (size_t(qrow) * p.hq + head[rb]) * DQK + 8 * half;
#pragma unroll
      for (int st = 0; st < S::KSTEPS; ++st)
        qf[rb][st] = valid[rb] ? *reinterpret_cast<const bf16x8*>(qsrc + 16 * st) : bf16x8{};
    }
  };
  if constexpr (!PACKED) load_q();

  // Loader geometry: load i of this wave fills LDS bytes [1 KB * gi, +1 KB) of
  // the K (or V) tile, gi = wave * IPW + i; lane l writes slot q = 64 gi + l,
  // i.e. row q / CPR, chunk position q % CPR, holding global chunk
  // (q % CPR) ^ swz(row). Everything but the gathered row is the same for
  // every tile, so each load's byte offset is precomputed once per lane; K
  // and V are below 4 GiB (checked at the boundary), so offsets are 32-bit.
  int key_rel[S::NROWS];      // tile-relative key of this lane's load i
  uint32_t lane_off[S::K_IPW + S::V_IPW];
#pragma unroll
  for (int i = 0; i < S::K_IPW; ++i) {
    const int q = (wave * S::K_IPW + i) * 64 + lane;
    const int r = q / S::KCPR;
    key_rel[i] = r;
    lane_off[i] = uint32_t(kvh * S::KROWB + (((q - r * S::KCPR) ^ swz<S::KCPR>(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < S::V_IPW; ++i) {
    const int q = (wave * S::V_IPW + i) * 64 + lane;
    const int r = q / S::VCPR;
    if (!S::SAME_ROWS) key_rel[S::K_IPW + i] = r;
    lane_off[S::K_IPW + i] = uint32_t(kvh * S::VROWB + (((q - r * S::VCPR) ^ swz<S::VCPR>(r)) << 4));
  }
  const uint32_t k_stride = uint32_t(hkv * S::KROWB);   // bytes per gathered K row
  const uint32_t v_stride = uint32_t(hkv * S::VROWB);
  int rows_cur[S::NROWS];   // gathered rows of this lane's keys, next tile to load
  int rows_nxt[S::NROWS];   // ... and the tile after it
  auto fetch_rows = [&](int j, int* rows) {
    const int key0 = kv_start + j * BN;
#pragma unroll
    for (int i = 0; i < S::NROWS; ++i) rows[i] = kv_row[min(key0 + key_rel[i], key_last)];
  };
  auto issue_tile = [&](char* stage, const int* rows) {
#pragma unroll
    for (int i = 0; i < S::K_IPW; ++i) {
      const char* src = kb + (uint32_t(rows[i]) * k_stride + lane_off[i]);
      load_lds16(src, stage + (wave * S::K_IPW + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::V_IPW; ++i) {
      const int grow = S::SAME_ROWS ? rows[i] : rows[S::K_IPW + i];
      const char* src = vb + (uint32_t(grow) * v_stride + lane_off[S::K_IPW + i]);
      load_lds16(src, stage + S::KBYTES + (wave * S::V_IPW + i) * 1024);
    }
  };

  // Per-lane LDS read offsets (relative to a stage).
  // K operand: row 32*kb + lrow, chunk 2*st + half.
  const int k_swz = swz<S::KCPR>(lrow);          // same for rows lrow and 32 + lrow
  const int k_off = lrow * S::KROWB;
  // V^T operand via transpose reads: lane (group g = lane/16, a = (lane%16)/4,
  // c = lane%4) reads row 16t + 4*half + a (+8), columns 32b + 16(g%2) + 4c .. +3.
  const int tr_a = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int tr_dv = 16 * ((lane >> 4) & 1) + 4 * tr_c;     // plus 32*b
  // Offsets of those reads for 16-key step 0; a row's swizzle depends only on
  // its index mod 16 (mod 8 for 8-chunk rows), so step t only adds 16 t rows,
  // a constant that the reads take as their immediate offset.
  int vt_off[2][S::DVB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int b = 0; b < S::DVB; ++b) {
      const int r = 4 * half + tr_a + 8 * h;
      const int dv = 32 * b + tr_dv;
      vt_off[h][b] = S::KBYTES + r * S::VROWB + (((dv >> 3) ^ swz<S::VCPR>(r)) << 4) + ((tr_c & 1) << 3);
    }

  f32x16 acc[RB][S::DVB];
  float m_run[RB], l_run[RB];   // running max of scale*log2(e)*s, and this lane's share of the sum
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int b = 0; b < S::DVB; ++b) acc[rb][b] = f32x16{};
    // A packed row can meet KV tiles it sees nothing of before its first
    // visible one: a finite start keeps exp2(s - m) at 0 for those (-inf - m),
    // where -inf - (-inf) would be NaN.
    m_run[rb] = PACKED ? -__FLT_MAX__ : -INFINITY;
    l_run[rb] = 0.0f;
  }
  const float c2 = p.scale_log2;

  // The keys of one item (of one run, for a pass): prologue, then the loop.
  auto walk = [&]() __attribute__((always_inline)) {
  // Prologue: rows of the first two KV tiles, then the first tile's data.
  fetch_rows(kv_begin, rows_cur);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  issue_tile(smem0, rows_cur);
  // Packed tiles: the slot window of the wave's rows. Both ends of the rows'
  // windows grow along the rows, so it runs from the first row's first slot
  // to the last valid row's last slot; KV tiles outside it are skipped.
  int w_lo = 0, w_hi = INT_MAX;
  if constexpr (PACKED) {
    static_assert(RB == 1, "the wave window reads one row block");
    load_q();
    if (packed_tile && wave_active) {
      const int last = min(31, n_rows * G - 1 - 32 * wave);
      w_lo = __builtin_amdgcn_readfirstlane(qlo[0]);
      w_hi = __builtin_amdgcn_readfirstlane(__shfl(qpos[0], last));
    }
  }
  if (kv_begin + 1 < kv_end) fetch_rows(kv_begin + 1, rows_cur);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  auto step = [&](int j, const char* stage, char* next) {
    // stage holds tile j; rows_cur holds tile j+1's rows.
    if (j + 1 < kv_end) issue_tile(next, rows_cur);
    if (j + 2 < kv_end) fetch_rows(j + 2, rows_nxt);

    if (wave_active && (!PACKED || (j * BN <= w_hi && j * BN + BN - 1 >= w_lo))) {
      // Opaque to the compiler on every tile, so that it adds each read's
      // constant in the read's immediate instead of keeping a register per
      // (step, column block) live across the loop.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < S::DVB; ++b) asm volatile("" : "+v"(vt_off[h][b]));
      // S^T = K Q^T for keys [32*kb, 32*kb + 32) of the tile; each K fragment
      // read from LDS feeds every row block.
      f32x16 s[RB][S::KB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb2 = 0; kb2 < S::KB; ++kb2) s[rb][kb2] = f32x16{};
      if constexpr (BN == kBlockN && DQK <= 128) {
        // K fragments one k-step ahead: the reads of step st + 1 are in flight
        // while step st's MFMAs run (the partial wait leaves them outstanding).
        // Not for 32-key tiles, nor for d_qk = 192, whose twelve Q fragments
        // leave no room: there the extra fragments spill or cost more than the
        // overlap gains.
        bf16x8 ka[2][S::KB];
#pragma unroll
        for (int kb2 = 0; kb2 < S::KB; ++kb2)
          ka[0][kb2] = *reinterpret_cast<const bf16x8*>(stage + k_off + 32 * kb2 * S::KROWB + ((half ^ k_swz) * 16));
#pragma unroll
        for (int st = 0; st < S::KSTEPS; ++st) {
          if (st + 1 < S::KSTEPS) {
            const int cpos = ((2 * (st + 1) + half) ^ k_swz) * 16;
#pragma unroll
            for (int kb2 = 0; kb2 < S::KB; ++kb2)
              ka[(st + 1) & 1][kb2] = *reinterpret_cast<const bf16x8*>(stage + k_off + 32 * kb2 * S::KROWB + cpos);
            __builtin_amdgcn_s_waitcnt(kWaitLgkmKB<S::KB>);   // this step's reads have landed
          } else {
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb2 = 0; kb2 < S::KB; ++kb2)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              if (rb_active[rb]) s[rb][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st & 1][kb2], qf[rb][st], s[rb][kb2], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int st = 0; st < S::KSTEPS; ++st) {
          const int cpos = ((2 * st + half) ^ k_swz) * 16;
#pragma unroll
          for (int kb2 = 0; kb2 < S::KB; ++kb2) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + k_off + 32 * kb2 * S::KROWB + cpos);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              if (rb_active[rb]) s[rb][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][st], s[rb][kb2], 0, 0, 0);
          }
        }
      }

      bf16x8 pb[RB][EXACT ? 1 : S::TS];
      float neg_m_rb[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (!rb_active[rb]) continue;
        if (j >= n_full) {
          const int key0 = kv_start + j * BN + 4 * half;
          if constexpr (BN == kBlockNShort) {
            // key0 + off > qpos exactly when off > qpos - key0 (key0 >= 0,
            // so the INT_MAX of rows past the tile cannot overflow): inline
            // constant offsets, one compare and one select per element. It
            // pays where most tiles are masked (short documents, -2%); with
            // 64-key tiles the other form timed slightly faster.
            // A packed row's window also has a first slot (lim_lo; <= 0, so
            // no bound, outside packed tiles). One form for both kinds of
            // tile: a branch between two copies costs the 32-key kernel 44
            // more bytes of spills.
            const int lim = qpos[rb] - key0;
            const int lim_lo = qlo[rb] - key0;
#pragma unroll
            for (int kb2 = 0; kb2 < S::KB; ++kb2)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int off = 32 * kb2 + 8 * (r >> 2) + (r & 3);
                if (off > lim || (PACKED && off < lim_lo)) s[rb][kb2][r] = -INFINITY;
              }
          } else {
#pragma unroll
            for (int kb2 = 0; kb2 < S::KB; ++kb2)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * kb2 + 8 * (r >> 2) + (r & 3);
                if (key > qpos[rb] || (PACKED && key < qlo[rb])) s[rb][kb2][r] = -INFINITY;
              }
          }
        }

        // This lane's half of the row maximum, as a tree of three-input maxima
        // (v_max3_f32: 32 values in 16 instructions, short chains).
        constexpr int NV = 16 * S::KB;
        float mv[NV];
#pragma unroll
        for (int kb2 = 0; kb2 < S::KB; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mv[16 * kb2 + r] = s[rb][kb2][r];
        int nv = NV;
#pragma unroll
        for (int round = 0; round < 6; ++round) {
          if (nv <= 1) break;
          const int n3 = nv / 3, rem = nv - 3 * n3;
#pragma unroll
          for (int i = 0; i < n3; ++i) mv[i] = fmaxf(mv[3 * i], fmaxf(mv[3 * i + 1], mv[3 * i + 2]));
          if (rem == 2) {
            mv[n3] = fmaxf(mv[3 * n3], mv[3 * n3 + 1]);
            nv = n3 + 1;
          } else if (rem == 1) {
            mv[n3] = mv[3 * n3];
            nv = n3 + 1;
          } else {
            nv = n3;
          }
        }
        const float m_half = mv[0] * c2;
        // A row is rescaled only when its maximum grows by more than the slack,
        // which a row can only do if one of its halves does: only then do the
        // halves exchange maxima. Each row decides on its own (its arithmetic
        // never depends on its neighbours); the wave skips the whole step when
        // no row needs it, which is the common case.
        if (__any(m_half > m_run[rb] + kRescaleSlack)) {
          const float m_tile = fmaxf(m_half, __shfl_xor(m_half, 32));
          const bool need = m_tile > m_run[rb] + kRescaleSlack;
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run[rb] - m_tile) : 1.0f;
#pragma unroll
          for (int b = 0; b < S::DVB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rb][b][r] *= alpha;
          l_run[rb] *= alpha;
          m_run[rb] = need ? m_tile : m_run[rb];
        }

        const float neg_m = -m_run[rb];
        neg_m_rb[rb] = neg_m;
        float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // independent partial sums
        if constexpr (!EXACT) {
#pragma unroll
          for (int kb2 = 0; kb2 < S::KB; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][kb2][r], c2, neg_m));
              ls[r & 3] += e;
              pb[rb][2 * kb2 + (r >> 3)][r & 7] = static_cast<__bf16>(e);
            }
        }
        l_run[rb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
      }

      // O^T += V^T P^T, 16 keys per MFMA: keys 16t + 4*half + {0..3, 8..11};
      // each V^T fragment feeds every row block. EXACT computes each 16-key
      // step's P here (exp, then the bf16 pair split) so that only one step's
      // pairs are live at a time.
#pragma unroll
      for (int t = 0; t < S::TS; ++t) {
        bf16x8 p_hi[RB], p_lo[RB];
        if constexpr (EXACT) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if (!rb_active[rb]) continue;
            u32x4 hw4, lw4;
            float lsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
              const int r = 8 * (t & 1) + i;
              const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][t >> 1][r], c2, neg_m_rb[rb]));
              const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][t >> 1][r + 1], c2, neg_m_rb[rb]));
              lsum += e0 + e1;
              unsigned hw, lw;
              split_pair(e0, e1, hw, lw);
              hw4[i >> 1] = hw;
              lw4[i >> 1] = lw;
            }
            l_run[rb] += lsum;
            p_hi[rb] = __builtin_bit_cast(bf16x8, hw4);
            p_lo[rb] = __builtin_bit_cast(bf16x8, lw4);
          }
        } else {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) p_hi[rb] = pb[rb][t];
        }
#pragma unroll
        for (int b = 0; b < S::DVB; ++b) {
          const int off0 = vt_off[0][b] + 16 * t * S::VROWB;
          const int off1 = vt_off[1][b] + 16 * t * S::VROWB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + off0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + off1));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if (!rb_active[rb]) continue;
            acc[rb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p_hi[rb], acc[rb][b], 0, 0, 0);
            if constexpr (EXACT)
              acc[rb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p_lo[rb], acc[rb][b], 0, 0, 0);
          }
        }
      }
    }

    // Tile j+1 (and tile j+2's rows) must have landed, and every wave must be
    // done with this stage before it is refilled.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < S::NROWS; ++i) rows_cur[i] = rows_nxt[i];
  };
  for (int j = kv_begin; j < kv_end; j += 2) {
    step(j, smem0, smem1);
    if (j + 1 < kv_end) step(j + 1, smem1, smem0);
  }
  };
  if constexpr (RANGED) {
    // A pass walks each run of the tile; the causal limit of every row is
    // also clamped to the run's end. The loop drains its copies and ends on
    // a barrier, so the next run's prologue may refill the ring.
    for (int r = 0; r < n_runs; ++r) {
      if (r > 0) {
        const int32_t* ru = runs + size_t(r) * 8;
        kv_start = ru[1];
        key_hi = ru[2];
        kv_end = ru[4];
        n_full = ru[5];
        key_last = key_hi - 1;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        qpos[rb] = valid[rb] ? min(q_glob0 + tok[rb], key_last) : INT_MAX;
      walk();
    }
  } else {
    walk();
  }

  static_assert(RB == 1, "the epilogue stages one 32-row block per wave");
  if (!wave_active) return;
  {
    // Recompute the lane's row, token and head from an opaque copy of the
    // lane id: otherwise the compiler keeps the address products it formed
    // from them before the tile loop live across it, and spills them (12 to
    // 28 bytes per lane in the 32-key and d_qk = 192 kernels).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    half = ln >> 5;
    lrow = ln & 31;
    const int row = 32 * wave + lrow;
    tok[0] = row / G;
    head[0] = kvh * G + (row - tok[0] * G);
    valid[0] = tok[0] < n_rows;
  }
  const float l_tot = l_run[0] + __shfl_xor(l_run[0], 32);
  const float inv = 1.0f / l_tot;
  if constexpr (RANGED) {
    // Merge into the running state: per row, this pass's (O, log2-sum-exp)
    // and the state's, weighted by 2^(lse2 - max) (THD_PASS_FIRST: the state
    // counts as empty). THD_PASS_LAST writes O (bf16; pad rows 0) and LSE
    // (natural log; pad rows +inf), otherwise the merged state. Each row of a
    // tile belongs to this one workgroup in a pass; the row's two lanes read
    // its lse2 in the same instruction before one of them stores the new one.
    if (!valid[0]) return;
    const bool first = (p.pass_flags & THD_PASS_FIRST) != 0;
    const bool last = (p.pass_flags & THD_PASS_LAST) != 0;
    const size_t orow = size_t(q_local0 + tok[0]) * p.hq + head[0];
    float* st_o = p.state + orow * DV;
    float* st_l = p.state + size_t(p.local) * p.hq * DV + orow;
    const bool own_any = l_tot > 0.0f;   // no run, or (never) no visible key
    const float own = own_any ? m_run[0] + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    const float ls = first ? -INFINITY : *st_l;
    const float mx = fmaxf(own, ls);
    float w_own = 0.0f, w_st = 0.0f, lnew = -INFINITY, norm = 0.0f;
    if (mx > -INFINITY) {
      w_own = own_any ? __builtin_amdgcn_exp2f(own - mx) : 0.0f;
      w_st = ls > -INFINITY ? __builtin_amdgcn_exp2f(ls - mx) : 0.0f;
      lnew = mx + __builtin_amdgcn_logf(w_own + w_st);
      norm = 1.0f / (w_own + w_st);
    }
    const float a_own = own_any ? w_own * inv * norm : 0.0f;   // weight of acc
    const float a_st = w_st * norm;
    const bool pad = last && q_glob0 + tok[0] >= p.doc_end[td[3]];
#pragma unroll
    for (int b = 0; b < S::DVB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * b + 8 * g + 4 * half;
        f32x4 o4;
        if (a_st != 0.0f) {
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(st_o + col);
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = __builtin_fmaf(acc[0][b][4 * g + e], a_own, s4[e] * a_st);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = acc[0][b][4 * g + e] * a_own;
        }
        if (last) {
          bf16x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(pad ? 0.0f : o4[e]);
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.o) + orow * DV + col) = out;
        } else {
          *reinterpret_cast<f32x4*>(st_o + col) = o4;
        }
      }
    if (half == 0) {
      if (last)
        p.lse[orow] = pad ? INFINITY : lnew * kLn2;
      else
        *st_l = lnew;
    }
    return;
  }
  if (part >= 0) {
    // Part of a split tile: its O normalised by its own sum, and its
    // log2-sum-exp, for the combine kernel.
    if (!valid[0]) return;
    const int rows = p.block_t * G;
    const int row = 32 * wave + lrow;
    float* base = p.partial + (size_t(part) * p.hkv + kvh) * size_t(fwd_partial_floats(p.block_t, G, DV));
    float* orow = base + size_t(row) * DV;
#pragma unroll
    for (int b = 0; b < S::DVB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = acc[0][b][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * b + 8 * g + 4 * half) = out;
      }
    if (half == 0) base[size_t(rows) * DV + row] = m_run[0] + __builtin_amdgcn_logf(l_tot);
    return;
  }
  // O leaves through LDS: each lane holds 4 columns of one row per (b, g),
  // which as global stores would write 16 bytes per row per instruction. The
  // wave writes its 32 rows into its own part of the ring (free once the last
  // tile's barrier has passed), 16-byte chunks XOR-swizzled by row, then
  // stores whole rows, 16 bytes per lane.
  char* region = (wave < 2 ? smem0 : smem1) + (wave & 1) * (32 * S::VROWB);
  const int qrow = PACKED ? pk_row[0] : q_local0 + tok[0];
  const bool real = PACKED ? pk_real[0] : tok[0] < n_real;
  const size_t orow_idx = size_t(qrow) * p.hq + head[0];
#pragma unroll
  for (int b = 0; b < S::DVB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 o4;
      bf16x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o4[e] = real ? acc[0][b][4 * g + e] * inv : 0.0f;   // pad rows get O = 0
        out[e] = static_cast<__bf16>(o4[e]);
      }
      const int chunk = (4 * b + g) ^ (lrow & (S::VCPR - 1));
      *reinterpret_cast<bf16x4*>(region + lrow * S::VROWB + chunk * 16 + half * 8) = out;
      if constexpr (EXACT)
        if (valid[0]) *reinterpret_cast<f32x4*>(p.o_f32 + orow_idx * DV + 32 * b + 8 * g + 4 * half) = o4;
    }
  if (half == 0 && valid[0])
    p.lse[orow_idx] = real ? (m_run[0] + __builtin_amdgcn_logf(l_tot)) * kLn2 : INFINITY;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __bf16* __restrict__ obase = static_cast<__bf16*>(p.o);
#pragma unroll
  for (int i = 0; i < 32 * S::VCPR / 64; ++i) {
    const int q = i * 64 + lane;
    const int r = q / S::VCPR;           // row within the wave's block
    const int c = q % S::VCPR;           // 16-byte chunk of the row
    const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(region + r * S::VROWB + ((c ^ (r & (S::VCPR - 1))) << 4));
    const int tok_r = __shfl(tok[0], r);
    const int head_r = __shfl(head[0], r);
    const int qrow_r = PACKED ? __shfl(qrow, r) : q_local0 + tok_r;
    if (tok_r < n_rows)
      *reinterpret_cast<bf16x8*>(obase + (size_t(qrow_r) * p.hq + head_r) * DV + 8 * c) = v8;
  }
}

// Merges the parts of split tiles: O = sum_p w_p O_p / sum_p w_p with
// w_p = 2^(lse_p - max lse), LSE = ln 2 * (max lse + log2 sum_p w_p). One
// thread per (split tile, kv head, row, 4 columns): every load is independent,
// so the pass is bandwidth-bound rather than latency-bound.
template <int DV>
__global__ __launch_bounds__(256) void thd_fwd_combine_kernel(FwdParams p) {
  constexpr int CPR = DV / 4;                // 4-float column groups per row
  const int G = p.group;
  const int rows = p.block_t * G;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_split = int64_t(p.hkv) * rows * CPR;
  if (idx >= per_split * p.n_splits) return;
  const int split = int(idx / per_split);
  int rem = int(idx - split * per_split);
  const int kvh = rem / (rows * CPR);
  rem -= kvh * rows * CPR;
  const int row = rem / CPR;
  const int col = (rem - row * CPR) * 4;
  const int32_t* sp = p.splits + size_t(split) * 4;
  const int tile = sp[0], first = sp[1], n_parts = sp[2];
  const int32_t* td = p.tiles + size_t(tile) * 8;
  const int tok = row / G;
  if (tok >= td[2]) return;                  // row past the tile's last token
  const bool pad = td[1] + tok >= p.doc_end[td[3]];   // written as O = 0, LSE = +inf
  const size_t slot_floats = size_t(fwd_partial_floats(p.block_t, G, DV));
  const float* base0 = p.partial + (size_t(first) * p.hkv + kvh) * slot_floats;
  const size_t part_stride = size_t(p.hkv) * slot_floats;
  float mx = -INFINITY;
  for (int q = 0; q < n_parts; ++q) mx = fmaxf(mx, base0[q * part_stride + size_t(rows) * DV + row]);
  float wsum = 0.0f;
  f32x4 acc = {};
  for (int q = 0; q < n_parts; ++q) {
    const float* base = base0 + q * part_stride;
    const float w = __builtin_amdgcn_exp2f(base[size_t(rows) * DV + row] - mx);
    wsum += w;
    const f32x4 v = *reinterpret_cast<const f32x4*>(base + size_t(row) * DV + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, v[e], acc[e]);
  }
  const float inv = 1.0f / wsum;
  const int head = kvh * G + (row - tok * G);
  const size_t orow = size_t(td[0] + tok) * p.hq + head;
  bf16x4 out;
  f32x4 o4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o4[e] = pad ? 0.0f : acc[e] * inv;
    out[e] = static_cast<__bf16>(o4[e]);
  }
  *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.o) + orow * DV + col) = out;
  if (p.o_f32 != nullptr) *reinterpret_cast<f32x4*>(p.o_f32 + orow * DV + col) = o4;
  if (col == 0) p.lse[orow] = pad ? INFINITY : (mx + __builtin_amdgcn_logf(wsum)) * kLn2;
}

template <int DQK, int DV>
int launch_pass(const FwdParams& p, void* stream) {
  // p.n_items workgroups per kv head: the pass's tiles, in p.pass_order.
  if (p.n_items == 0) return int(hipSuccess);
  hipLaunchKernelGGL((thd_fwd_kernel<DQK, DV, false, kBlockN, true>),
                     dim3(unsigned(int64_t(p.n_items) * p.hkv)), dim3(kFwdThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return int(hipGetLastError());
}

template <int DQK, int DV, int BN>
int launch(const FwdParams& p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(int64_t(p.n_items) * p.hkv));
  if (p.packed) {
    if (p.o_f32 != nullptr)
      hipLaunchKernelGGL((thd_fwd_kernel<DQK, DV, true, BN, false, true>), grid, dim3(kFwdThreads), 0, st, p);
    else
      hipLaunchKernelGGL((thd_fwd_kernel<DQK, DV, false, BN, false, true>), grid, dim3(kFwdThreads), 0, st, p);
  } else if (p.o_f32 != nullptr) {
    hipLaunchKernelGGL((thd_fwd_kernel<DQK, DV, true, BN>), grid, dim3(kFwdThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((thd_fwd_kernel<DQK, DV, false, BN>), grid, dim3(kFwdThreads), 0, st, p);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.n_splits == 0) return int(err);
  const int64_t threads = int64_t(p.n_splits) * p.hkv * p.block_t * p.group * (DV / 4);
  hipLaunchKernelGGL((thd_fwd_combine_kernel<DV>), dim3(unsigned((threads + 255) / 256)),
                     dim3(256), 0, st, p);
  return int(hipGetLastError());
}

// Workspace of thd_attn_fwd_noalloc: the split tiles' partial results live in
// this file-scope array instead of a caller's buffer. Each device that runs the
// library holds its own copy until the process ends. In host code the name
// only stands for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device (looked up once per
// device, on that device's first call).
static __device__ __align__(256) char scratch[kFwdStaticScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device id; null until looked up

}  // namespace

int fwd_static_scratch(int device, void** ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0) return int(hipErrorInvalidDevice);
  if (size_t(device) >= g_scratch_ptr.size()) g_scratch_ptr.resize(size_t(device) + 1, nullptr);
  if (g_scratch_ptr[size_t(device)] == nullptr) {
    // The caller has made `device` current: the address is that device's copy.
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return int(err);
    if (p == nullptr) return int(hipErrorInvalidSymbol);
    g_scratch_ptr[size_t(device)] = p;
  }
  *ptr = g_scratch_ptr[size_t(device)];
  return int(hipSuccess);
}

bool fwd_supported(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

bool fwd_block_n_supported(int d_qk, int block_n) {
  // 32-key tiles are not built for d_qk = 192: at 168 registers per lane the
  // MLA kernel spills.
  return block_n == kBlockN || (block_n == kBlockNShort && d_qk <= 128);
}

int fwd_workgroups_per_cu(int block_n) {
  return block_n == kBlockNShort ? kFwdOccupancy<kBlockNShort> : kFwdOccupancy<kBlockN>;
}

int launch_fwd_pass(const FwdParams& p, int d_qk, int d_v, void* stream) {
  if (d_qk == 64 && d_v == 64) return launch_pass<64, 64>(p, stream);
  if (d_qk == 128 && d_v == 128) return launch_pass<128, 128>(p, stream);
  if (d_qk == 192 && d_v == 128) return launch_pass<192, 128>(p, stream);
  return int(hipErrorInvalidValue);
}

int launch_fwd(const FwdParams& p, int d_qk, int d_v, void* stream) {
  const bool short_tiles = p.block_n == kBlockNShort;
  if (d_qk == 64 && d_v == 64)
    return short_tiles ? launch<64, 64, kBlockNShort>(p, stream) : launch<64, 64, kBlockN>(p, stream);
  if (d_qk == 128 && d_v == 128)
    return short_tiles ? launch<128, 128, kBlockNShort>(p, stream) : launch<128, 128, kBlockN>(p, stream);
  if (d_qk == 192 && d_v == 128 && !short_tiles) return launch<192, 128, kBlockN>(p, stream);
  return int(hipErrorInvalidValue);
}

}  // namespace thd
