// Backward kernels: gradients of causal + EOD-reset attention for one rank,
// against rank-major gathered K/V (gfx950, bf16 MFMA, fp32 accumulate).
//
// With P = softmax of the visible scores (recomputed from the forward's LSE)
// and dO the upstream gradient:
//   dP = dO V^T,  D = rowsum(P * dP),  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q,  dV = P^T dO   (dK, dV summed over the G heads of a kv head).
// D equals rowsum(dO * O) for the exact O; it is computed from P and dP in
// fp32 rather than from the forward's bf16 O, whose rounding would otherwise
// dominate the gradients' error.
// The attention is the one of "kvallgather cp thd load balance" (Ascend/
// MindSpeed, "What this PR does / why we need it?"); the backward of the
// all-gather is a reduce-scatter of dK/dV, so this rank's dK/dV are partial
// sums in the gathered layout.
//
// Three launches, no atomics (results are deterministic):
//   1. thd_bwd_dq_kernel<delta = true>: D for every local row and q head;
//   2. thd_bwd_dkdv_kernel (below);
//   3. thd_bwd_dq_kernel<delta = false>: dQ. Both dQ-kernel passes run one
//      workgroup per (query tile, kv head), laid out like the forward kernel:
//      K and V tiles stream through a two-stage LDS ring, S^T = K Q^T and
//      dP^T = V dO^T on MFMA, then (second pass) dQ^T += K^T dS^T with the
//      K^T operand read by ds_read_b64_tr_b16;
//   dS (and P in dV = P^T dO) enter their products as a pair of bf16 values
//   (hi, lo = x - hi), so their rounding error is ~2^-17 instead of bf16's
//   2^-9: the gradients are then limited by fp32 accumulation only;
//   thd_bwd_dkdv_kernel: one workgroup (2 waves, 32 keys each) per
//      (64-key tile, kv head). The key tiles cover every key once; the query
//      tiles that see a key tile are a suffix of its document's tiles, walked
//      in 32-row blocks (token-major rows: all G heads of a kv head) through a
//      two-stage LDS ring. S = Q K^T and dP = dO V^T leave each lane with one
//      key and 16 rows, which is the A-operand layout of P^T and dS^T, so
//      dV += P^T dO and dK += dS^T Q take their B operands from the row-major
//      dO and Q blocks with transpose reads. Tiles no local query sees write
//      zeros.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "internal.h"

namespace thd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaitVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0)
constexpr int BN = kBlockN;

// 16-byte global -> LDS copy: lane i's 16 bytes land at lds + 16 * i (lds is
// wave-uniform). Kept as a function taking a named pointer: handing the
// builtin a pointer expression directly inside a kernel template makes the
// host pass drop that kernel's launch stub.
__device__ __forceinline__ void load_lds16(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
}

template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (r >> 1) & 7;
  }
}

__device__ __forceinline__ bf16x8 tr_pair(const char* base, int off0, int off1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Byte offset of the 8-byte piece (row, col .. col+3) in a row-major tile with
// ROWB-byte rows whose 16-byte chunks are swizzled by swz<CPR>(row).
template <int CPR, int ROWB>
__device__ __forceinline__ int piece(int row, int col) {
  return row * ROWB + (((col >> 3) ^ swz<CPR>(row)) << 4) + ((col & 4) << 1);
}

// ---------------------------------------------------------------- dQ
template <int DQK, int DV>
struct DqShape {
  static constexpr int KCPR = DQK / 8, VCPR = DV / 8;
  static constexpr int KROWB = DQK * 2, VROWB = DV * 2;
  static constexpr int KBYTES = BN * KROWB, VBYTES = BN * VROWB, STAGE = KBYTES + VBYTES;
  static constexpr int K_IPW = BN * KCPR / 64 / kWaves;
  static constexpr int V_IPW = BN * VCPR / 64 / kWaves;
  static constexpr bool SAME_ROWS = (KCPR == VCPR);
  static constexpr int NROWS = SAME_ROWS ? K_IPW : K_IPW + V_IPW;
  static constexpr int KSTEPS = DQK / 16, VSTEPS = DV / 16, DQB = DQK / 32;
};

template <int DQK, int DV, bool DELTA>
__global__ __launch_bounds__(kWaves * 64, DQK > 128 ? 1 : 2) void thd_bwd_dq_kernel(BwdParams p) {
  using S = DqShape<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * S::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int lrow = lane & 31;

  const int kvh = blockIdx.x % p.hkv;
  const int tile = blockIdx.x / p.hkv;
  const int32_t* td = p.tiles + size_t(tile) * 8;
  const int q_local0 = td[0], q_glob0 = td[1], n_rows = td[2], kv_start = td[5];
  const int n_kv = td[6], n_full = td[7];
  const int key_last = q_glob0 + n_rows - 1;

  const int G = p.group;
  const int row = wave * 32 + lrow;
  const int tok = row / G;
  const int head = kvh * G + (row - tok * G);
  const bool valid = tok < n_rows;
  const int qpos = valid ? q_glob0 + tok : INT_MAX;
  const bool wave_active = (wave * 32) / G < n_rows;
  const size_t qrow_idx = size_t(q_local0 + tok) * p.hq + head;

  bf16x8 qf[S::KSTEPS];
  bf16x8 df[S::VSTEPS];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + qrow_idx * DQK + 8 * half;
    const __bf16* drow = static_cast<const __bf16*>(p.d_o) + qrow_idx * DV + 8 * half;
#pragma unroll
    for (int st = 0; st < S::KSTEPS; ++st)
      qf[st] = valid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * st) : bf16x8{};
#pragma unroll
    for (int st = 0; st < S::VSTEPS; ++st)
      df[st] = valid ? *reinterpret_cast<const bf16x8*>(drow + 16 * st) : bf16x8{};
  }
  const float lse2 = valid ? p.lse[qrow_idx] * kLog2e : 0.0f;
  const float dl = (!DELTA && valid) ? p.delta[qrow_idx] : 0.0f;
  float dsum = 0.0f;   // delta pass: this lane's share of rowsum(P * dP)

  const char* __restrict__ kb = static_cast<const char*>(p.k);
  const char* __restrict__ vb = static_cast<const char*>(p.v);
  const int hkv = p.hkv;
  int rows_cur[S::NROWS];
  int rows_nxt[S::NROWS];
  auto key_row = [&](int i) -> int {
    if (i < S::K_IPW) return ((wave * S::K_IPW + i) * 64 + lane) / S::KCPR;
    return ((wave * S::V_IPW + (i - S::K_IPW)) * 64 + lane) / S::VCPR;
  };
  auto fetch_rows = [&](int j, int* rows) {
    const int key0 = kv_start + j * BN;
#pragma unroll
    for (int i = 0; i < S::NROWS; ++i) rows[i] = p.kv_row[min(key0 + key_row(i), key_last)];
  };
  auto issue_tile = [&](int j, const int* rows) {
    char* stage = smem + (j & 1) * S::STAGE;
#pragma unroll
    for (int i = 0; i < S::K_IPW; ++i) {
      const int q = (wave * S::K_IPW + i) * 64 + lane;
      const int r = q / S::KCPR;
      const int c = (q - r * S::KCPR) ^ swz<S::KCPR>(r);
      const char* src = kb + (size_t(rows[i]) * hkv + kvh) * S::KROWB + c * 16;
      load_lds16(src, stage + (wave * S::K_IPW + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::V_IPW; ++i) {
      const int q = (wave * S::V_IPW + i) * 64 + lane;
      const int r = q / S::VCPR;
      const int c = (q - r * S::VCPR) ^ swz<S::VCPR>(r);
      const int grow = S::SAME_ROWS ? rows[i] : rows[S::K_IPW + i];
      const char* src = vb + (size_t(grow) * hkv + kvh) * S::VROWB + c * 16;
      load_lds16(src, stage + S::KBYTES + (wave * S::V_IPW + i) * 1024);
    }
  };

  const int tr_a = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  f32x16 acc[S::DQB];
#pragma unroll
  for (int b = 0; b < S::DQB; ++b) acc[b] = f32x16{};
  const float c2 = p.scale_log2;

  fetch_rows(0, rows_cur);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  issue_tile(0, rows_cur);
  if (n_kv > 1) fetch_rows(1, rows_cur);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) issue_tile(j + 1, rows_cur);
    if (j + 2 < n_kv) fetch_rows(j + 2, rows_nxt);
    const char* stage = smem + (j & 1) * S::STAGE;
    if (wave_active) {
      f32x16 s[2] = {f32x16{}, f32x16{}};
      f32x16 dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int r = 32 * kb2 + lrow;
#pragma unroll
        for (int st = 0; st < S::KSTEPS; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              stage + r * S::KROWB + (((2 * st + half) ^ swz<S::KCPR>(r)) << 4));
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb2], 0, 0, 0);
        }
#pragma unroll
        for (int st = 0; st < S::VSTEPS; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              stage + S::KBYTES + r * S::VROWB + (((2 * st + half) ^ swz<S::VCPR>(r)) << 4));
          dp[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[st], dp[kb2], 0, 0, 0);
        }
      }
      const bool masked = j >= n_full;
      const int key0 = kv_start + j * BN + 4 * half;
      // dS as a bf16 pair (hi + lo): its rounding stays ~2^-17 relative.
      bf16x8 dsb[4], dsl[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb2 + 8 * (r >> 2) + (r & 3);
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][r], c2, -lse2));
          if (masked && key > qpos) pr = 0.0f;
          if constexpr (DELTA) {
            dsum = __builtin_fmaf(pr, dp[kb2][r], dsum);
          } else {
            const float ds = pr * (dp[kb2][r] - dl);
            const __bf16 hi = static_cast<__bf16>(ds);
            dsb[2 * kb2 + (r >> 3)][r & 7] = hi;
            dsl[2 * kb2 + (r >> 3)][r & 7] = static_cast<__bf16>(ds - static_cast<float>(hi));
          }
        }
      // dQ^T += K^T dS^T: K^T rows (dims) 32b + lane%32, keys 16t + 4*half + {0..3, 8..11}.
#pragma unroll
      for (int t = 0; t < (DELTA ? 0 : 4); ++t) {
        const int r0 = 16 * t + 4 * half + tr_a;
#pragma unroll
        for (int b = 0; b < S::DQB; ++b) {
          const int col = 32 * b + tr_col;
          const bf16x8 a = tr_pair(stage, piece<S::KCPR, S::KROWB>(r0, col),
                                   piece<S::KCPR, S::KROWB>(r0 + 8, col));
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[t], acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsl[t], acc[b], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < S::NROWS; ++i) rows_cur[i] = rows_nxt[i];
  }

  if constexpr (DELTA) {
    if (!wave_active) return;
    const float total = dsum + __shfl_xor(dsum, 32);
    if (valid && half == 0) p.delta[qrow_idx] = total;
    return;
  }
  if (!valid) return;
  float* dq = p.dq + qrow_idx * DQK;
#pragma unroll
  for (int b = 0; b < S::DQB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = acc[b][4 * g + e] * p.scale;
      *reinterpret_cast<f32x4*>(dq + 32 * b + 8 * g + 4 * half) = out;
    }
}

// ---------------------------------------------------------------- dK, dV
constexpr int kDkvWaves = 2;
constexpr int kRowsPerBlock = 32;

template <int DQK, int DV>
struct DkvShape {
  static constexpr int KCPR = DQK / 8, VCPR = DV / 8;
  static constexpr int KROWB = DQK * 2, VROWB = DV * 2;
  static constexpr int KBYTES = BN * KROWB, VBYTES = BN * VROWB;
  static constexpr int QBYTES = kRowsPerBlock * KROWB, OBYTES = kRowsPerBlock * VROWB;
  // stage: Q block, dO block, then per-row lse (log2 units), D, and query position
  static constexpr int STAGE = QBYTES + OBYTES + 3 * kRowsPerBlock * 4;
  static constexpr int KV_BYTES = KBYTES + VBYTES;
  static constexpr int K_IPW = BN * KCPR / 64 / kDkvWaves;     // K tile loads per wave
  static constexpr int V_IPW = BN * VCPR / 64 / kDkvWaves;
  static constexpr int Q_IPW = kRowsPerBlock * KCPR / 64 / kDkvWaves;
  static constexpr int O_IPW = kRowsPerBlock * VCPR / 64 / kDkvWaves;
  static constexpr int KSTEPS = DQK / 16, VSTEPS = DV / 16, DQB = DQK / 32, DVB = DV / 32;
  static_assert(kRowsPerBlock * KCPR % (64 * kDkvWaves) == 0, "Q block must split evenly");
  static_assert(kRowsPerBlock * VCPR % (64 * kDkvWaves) == 0, "dO block must split evenly");
};

template <int DQK, int DV>
__global__ __launch_bounds__(kDkvWaves * 64, 1) void thd_bwd_dkdv_kernel(BwdParams p) {
  using S = DkvShape<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) char smem[S::KV_BYTES + 2 * S::STAGE];
  char* const kv_lds = smem;
  char* const ring = smem + S::KV_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int lrow = lane & 31;

  const int kvh = blockIdx.x % p.hkv;
  const int kt = blockIdx.x / p.hkv;
  const int32_t* kd = p.kvtiles + size_t(kt) * 8;
  const int ks = kd[1], nk = kd[2], qb = kd[3], qe = kd[4];
  const int G = p.group;
  const int hkv = p.hkv;
  const int hq = p.hq;
  const char* __restrict__ kb = static_cast<const char*>(p.k);
  const char* __restrict__ vb = static_cast<const char*>(p.v);
  const char* __restrict__ qbase = static_cast<const char*>(p.q);
  const char* __restrict__ obase = static_cast<const char*>(p.d_o);

  // K and V of this key tile (keys past the tile's end are clamped to its last
  // key; they are masked out below and never stored).
  {
#pragma unroll
    for (int i = 0; i < S::K_IPW; ++i) {
      const int q = (wave * S::K_IPW + i) * 64 + lane;
      const int r = q / S::KCPR;
      const int c = (q - r * S::KCPR) ^ swz<S::KCPR>(r);
      const int grow = p.kv_row[ks + min(r, nk - 1)];
      const char* src = kb + (size_t(grow) * hkv + kvh) * S::KROWB + c * 16;
      load_lds16(src, kv_lds + (wave * S::K_IPW + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::V_IPW; ++i) {
      const int q = (wave * S::V_IPW + i) * 64 + lane;
      const int r = q / S::VCPR;
      const int c = (q - r * S::VCPR) ^ swz<S::VCPR>(r);
      const int grow = p.kv_row[ks + min(r, nk - 1)];
      const char* src = vb + (size_t(grow) * hkv + kvh) * S::VROWB + c * 16;
      load_lds16(src, kv_lds + S::KBYTES + (wave * S::V_IPW + i) * 1024);
    }
  }

  // Row blocks: query tile t in [qb, qe), block sb of its n_rows * G rows.
  struct Block {
    int t, sb;
  };
  auto rows_of = [&](int t) { return p.tiles[size_t(t) * 8 + 2] * G; };
  auto next_block = [&](Block b) -> Block {
    if ((b.sb + 1) * kRowsPerBlock < rows_of(b.t)) return Block{b.t, b.sb + 1};
    return Block{b.t + 1, 0};
  };
  // Source row (index into [T_local * Hq]) of block row x; rows past the tile's
  // end are clamped to its last row (and masked out by their query position).
  auto src_row = [&](Block b, int x, int* qpos) -> size_t {
    const int32_t* td = p.tiles + size_t(b.t) * 8;
    const int n_r = td[2] * G;
    const int ri = b.sb * kRowsPerBlock + x;
    const int rc = min(ri, n_r - 1);
    const int tok = rc / G;
    if (qpos) *qpos = ri < n_r ? td[1] + tok : -1;
    return size_t(td[0] + tok) * hq + kvh * G + (rc - tok * G);
  };
  auto issue_block = [&](Block b, int slot) {
    char* stage = ring + slot * S::STAGE;
#pragma unroll
    for (int i = 0; i < S::Q_IPW; ++i) {
      const int q = (wave * S::Q_IPW + i) * 64 + lane;
      const int r = q / S::KCPR;
      const int c = (q - r * S::KCPR) ^ swz<S::KCPR>(r);
      const char* src = qbase + src_row(b, r, nullptr) * S::KROWB + c * 16;
      load_lds16(src, stage + (wave * S::Q_IPW + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::O_IPW; ++i) {
      const int q = (wave * S::O_IPW + i) * 64 + lane;
      const int r = q / S::VCPR;
      const int c = (q - r * S::VCPR) ^ swz<S::VCPR>(r);
      const char* src = obase + src_row(b, r, nullptr) * S::VROWB + c * 16;
      load_lds16(src, stage + S::QBYTES + (wave * S::O_IPW + i) * 1024);
    }
    if (wave == 0 && lane < kRowsPerBlock) {
      int qpos;
      const size_t sr = src_row(b, lane, &qpos);
      float* rowinfo = reinterpret_cast<float*>(stage + S::QBYTES + S::OBYTES);
      rowinfo[lane] = p.lse[sr] * kLog2e;
      rowinfo[kRowsPerBlock + lane] = p.delta[sr];
      reinterpret_cast<int*>(rowinfo)[2 * kRowsPerBlock + lane] = qpos;
    }
  };

  f32x16 dk[S::DQB], dv[S::DVB];
#pragma unroll
  for (int b = 0; b < S::DQB; ++b) dk[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < S::DVB; ++b) dv[b] = f32x16{};

  const int key_rel = wave * 32 + lrow;            // this lane's key within the tile
  const int key = ks + key_rel;
  const bool key_ok = key_rel < nk;
  const float c2 = p.scale_log2;
  const int tr_a = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const char* kt_lds = kv_lds + key_rel * S::KROWB;
  const char* vt_lds = kv_lds + S::KBYTES + key_rel * S::VROWB;

  Block cur{qb, 0};
  if (qb < qe) issue_block(cur, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  for (int it = 0; cur.t < qe; ++it) {
    const Block nxt = next_block(cur);
    if (nxt.t < qe) issue_block(nxt, (it + 1) & 1);
    const char* stage = ring + (it & 1) * S::STAGE;

    // S = Q K^T and dP = dO V^T: lane holds key lane%32, rows 8(r/4) + 4*half + r%4.
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < S::KSTEPS; ++st) {
      const int ch = 2 * st + half;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + lrow * S::KROWB + ((ch ^ swz<S::KCPR>(lrow)) << 4));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(kt_lds + ((ch ^ swz<S::KCPR>(key_rel)) << 4));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, s, 0, 0, 0);
    }
#pragma unroll
    for (int st = 0; st < S::VSTEPS; ++st) {
      const int ch = 2 * st + half;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + S::QBYTES + lrow * S::VROWB + ((ch ^ swz<S::VCPR>(lrow)) << 4));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(vt_lds + ((ch ^ swz<S::VCPR>(key_rel)) << 4));
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, dp, 0, 0, 0);
    }
    const float* rowinfo = reinterpret_cast<const float*>(stage + S::QBYTES + S::OBYTES);
    bf16x8 pt[2], ptl[2], dst[2], dsl[2];   // P and dS as bf16 pairs (hi + lo)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r0 = 8 * g + 4 * half;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(rowinfo + r0);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(rowinfo + kRowsPerBlock + r0);
      const i32x4 q4 = *reinterpret_cast<const i32x4*>(rowinfo + 2 * kRowsPerBlock + r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -l4[e]));
        if (!key_ok || key > q4[e]) pr = 0.0f;
        const __bf16 phi = static_cast<__bf16>(pr);
        pt[r >> 3][r & 7] = phi;
        ptl[r >> 3][r & 7] = static_cast<__bf16>(pr - static_cast<float>(phi));
        const float ds = pr * (dp[r] - d4[e]);
        const __bf16 hi = static_cast<__bf16>(ds);
        dst[r >> 3][r & 7] = hi;
        dsl[r >> 3][r & 7] = static_cast<__bf16>(ds - static_cast<float>(hi));
      }
    }
    // dV += P^T dO and dK += dS^T Q; B operands: rows 16t + 4*half + {0..3, 8..11}.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 16 * t + 4 * half + tr_a;
#pragma unroll
      for (int b = 0; b < S::DVB; ++b) {
        const int col = 32 * b + tr_col;
        const bf16x8 o8 = tr_pair(stage + S::QBYTES, piece<S::VCPR, S::VROWB>(r0, col),
                                  piece<S::VCPR, S::VROWB>(r0 + 8, col));
        dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pt[t], o8, dv[b], 0, 0, 0);
        dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ptl[t], o8, dv[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < S::DQB; ++b) {
        const int col = 32 * b + tr_col;
        const bf16x8 q8 = tr_pair(stage, piece<S::KCPR, S::KROWB>(r0, col),
                                  piece<S::KCPR, S::KROWB>(r0 + 8, col));
        dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dst[t], q8, dk[b], 0, 0, 0);
        dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsl[t], q8, dk[b], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    cur = nxt;
  }

  // Store: lane holds dims 32b + lane%32 of keys 32*wave + 8(r/4) + 4*half + r%4.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = wave * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
    if (kr >= nk) continue;
    const size_t grow = size_t(p.kv_row[ks + kr]) * hkv + kvh;
#pragma unroll
    for (int b = 0; b < S::DQB; ++b) p.dk[grow * DQK + 32 * b + lrow] = dk[b][r] * p.scale;
#pragma unroll
    for (int b = 0; b < S::DVB; ++b) p.dv[grow * DV + 32 * b + lrow] = dv[b][r];
  }
}

template <int DQK, int DV>
int launch(const BwdParams& p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 q_grid(unsigned(int64_t(p.n_tiles) * p.hkv));
  hipLaunchKernelGGL((thd_bwd_dq_kernel<DQK, DV, true>), q_grid, dim3(kWaves * 64), 0, st, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return int(err);
  hipLaunchKernelGGL((thd_bwd_dkdv_kernel<DQK, DV>), dim3(unsigned(int64_t(p.n_kvtiles) * p.hkv)),
                     dim3(kDkvWaves * 64), 0, st, p);
  err = hipGetLastError();
  if (err != hipSuccess) return int(err);
  hipLaunchKernelGGL((thd_bwd_dq_kernel<DQK, DV, false>), q_grid, dim3(kWaves * 64), 0, st, p);
  return int(hipGetLastError());
}

}  // namespace

bool bwd_supported(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

int launch_bwd(const BwdParams& p, int d_qk, int d_v, void* stream) {
  if (d_qk == 64 && d_v == 64) return launch<64, 64>(p, stream);
  if (d_qk == 128 && d_v == 128) return launch<128, 128>(p, stream);
  if (d_qk == 192 && d_v == 128) return launch<192, 128>(p, stream);
  return int(hipErrorInvalidValue);
}

}  // namespace thd
