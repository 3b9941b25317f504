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
// Three launches, no atomics (results are deterministic), or two when the
// forward's exact fp32 O is given (dQ first, computing D = rowsum(dO * O) per
// row from it, then dK/dV):
//   1. thd_bwd_dq_kernel<delta = true>: D for every local row and q head;
//   2. thd_bwd_dkdv_kernel (below);
//   3. thd_bwd_dq_kernel<delta = false>: dQ. Both dQ-kernel passes run one
//      workgroup per (query tile, kv head), laid out like the forward kernel:
//      K and V tiles stream through a two-stage LDS ring, S^T = K Q^T and
//      dP^T = V dO^T on MFMA, then (second pass) dQ^T += K^T dS^T with the
//      K^T operand read by ds_read_b64_tr_b16;
//   dS (and P in dV = P^T dO) enter their products as a pair of bf16 values
//   (hi, lo = x - hi), so their rounding error is ~2^-17 instead of bf16's
//   2^-9: the gradients are then limited by fp32 accumulation only. (With dS
//   in plain bf16 the backward ran 12% faster, but dK, which sums over the G
//   heads of a kv head, reached max-abs 0.027 against fp64 at G = 64 and 128,
//   beyond the 2e-2 bound);
//   thd_bwd_dkdv_kernel: one workgroup (4 waves, 16 keys each) per
//      (64-key tile, kv head). The key tiles cover every key once; the query
//      tiles that see a key tile are a suffix of its document's tiles, walked
//      in 32-row blocks (token-major rows: all G heads of a kv head) through a
//      three-stage LDS ring. S = Q K^T and dP = dO V^T on 16x16x32 MFMA leave
//      each lane with one key and 8 rows, which is the A-operand layout of P^T
//      and dS^T, so dV += P^T dO and dK += dS^T Q take their B operands from
//      the row-major dO and Q blocks with transpose reads. Tiles no local
//      query sees write zeros. dK and dV are stored in fp32, or rounded to
//      bf16 (nearest even) when the caller asks for half the bytes in the
//      reduce-scatter.
// Dispatch order: dQ-kernel workgroups take query tiles in the plan's order
// (most KV tiles first), dK/dV workgroups key tiles by the local query tokens
// that see them (most first). Each workgroup writes only its own rows, so the
// order changes no result, only how evenly the CUs finish.
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(4))) const int32_t cint32_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaitVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;    // s_waitcnt lgkmcnt(0)
constexpr int kWaitLgkm1 = 0xC17F;    // s_waitcnt lgkmcnt(1)
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

// Returns x unchanged, hidden from the optimiser: a mask applied to the result
// in the same basic block survives, so instruction selection can see that a
// product fits a 24-bit multiply (full rate, where a 32-bit one is quarter rate).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
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
  // Products of S^T and dP^T in issue order: operand n = 4 * step + w, with
  // w = (K, keys 0-31), (V, keys 0-31), (K, keys 32-63), (V, keys 32-63).
  static constexpr int NSTEPS = KSTEPS > VSTEPS ? KSTEPS : VSTEPS;
  static constexpr bool has_op(int n) { return (n & 1) ? (n >> 2) < VSTEPS : (n >> 2) < KSTEPS; }
  static constexpr int next_op(int n) {
    for (int m = n + 1; m < 4 * NSTEPS; ++m)
      if (has_op(m)) return m;
    return -1;
  }
  static constexpr int op_index(int n) {
    int k = 0;
    for (int m = 0; m < n; ++m) k += has_op(m) ? 1 : 0;
    return k;
  }
};

// Two workgroups per CU, except the d_qk = 192 dQ pass: its Q and dO
// fragments, six dQ accumulators and the S and dP tiles need about 430
// registers (one workgroup per CU). Its D pass, without dQ, fits two.
template <int DQK, int DV, bool DELTA>
__global__ __launch_bounds__(kWaves * 64, DQK > 128 && !DELTA ? 1 : 2) void thd_bwd_dq_kernel(BwdParams p) {
  using S = DqShape<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * S::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int lrow = lane & 31;

  const int kvh = blockIdx.x % p.hkv;
  // Query tiles go out with the most KV tiles first (the plan's order), as
  // in the forward, so the longest walks do not start last.
  const int tile = ((const cint32_t*)p.order)[blockIdx.x / p.hkv];
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
  float dl = 0.0f;
  if constexpr (!DELTA) {
    if (p.o_f32 != nullptr) {
      // D = rowsum(dO * O) from the forward's exact fp32 O: this lane's dims
      // are those of its dO fragments, the other half's are in lane ^ 32.
      // Written (with lse2) for the dK/dV kernel, which runs after this one.
      float part = 0.0f;
      if (valid) {
        const float* orow = p.o_f32 + qrow_idx * DV + 8 * half;
#pragma unroll
        for (int st = 0; st < S::VSTEPS; ++st) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(orow + 16 * st);
          const f32x4 b = *reinterpret_cast<const f32x4*>(orow + 16 * st + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            part = __builtin_fmaf(a[e], static_cast<float>(df[st][e]), part);
            part = __builtin_fmaf(b[e], static_cast<float>(df[st][4 + e]), part);
          }
        }
      }
      dl = part + __shfl_xor(part, 32);
      if (valid && half == 0) {
        p.delta[qrow_idx] = dl;
        p.lse2[qrow_idx] = lse2;
      }
    } else if (valid) {
      dl = p.delta[qrow_idx];
    }
  }
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
      // The four products (K and V of each 32-key half) advance one k-step at
      // a time, and each operand is read from LDS one product ahead of its
      // MFMA: the partial wait leaves that read in flight while the MFMA
      // issues, instead of exposing every read's latency. Not at d_qk = 192,
      // where the second operand buffer spills.
      if constexpr (DQK <= 128) {
        auto frag = [&](int n) -> bf16x8 {
          const int st = n >> 2, w = n & 3, r = 32 * (w >> 1) + lrow;
          if (w & 1)
            return *reinterpret_cast<const bf16x8*>(
                stage + S::KBYTES + r * S::VROWB + (((2 * st + half) ^ swz<S::VCPR>(r)) << 4));
          return *reinterpret_cast<const bf16x8*>(
              stage + r * S::KROWB + (((2 * st + half) ^ swz<S::KCPR>(r)) << 4));
        };
        bf16x8 fb[2];
        fb[0] = frag(0);
#pragma unroll
        for (int n = 0; n < 4 * S::NSTEPS; ++n) {
          if (!S::has_op(n)) continue;
          const int nx = S::next_op(n);
          if (nx >= 0) {
            fb[(S::op_index(n) + 1) & 1] = frag(nx);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm1);
          } else {
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
          }
          __builtin_amdgcn_sched_barrier(0);
          const int st = n >> 2, w = n & 3;
          const bf16x8 a = fb[S::op_index(n) & 1];
          if (w & 1)
            dp[w >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[st], dp[w >> 1], 0, 0, 0);
          else
            s[w >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[w >> 1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
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
      }
      // Key key0 + off lies past this lane's row exactly when off > lim; lim
      // is INT_MAX on tiles before n_full, which every row sees whole (and
      // qpos - key0 cannot overflow: key0 >= 0). The offsets are inline
      // constants, so the test is one compare and one select per element.
      const int key0 = kv_start + j * BN + 4 * half;
      int lim = j >= n_full ? qpos - key0 : INT_MAX;
      asm volatile("" : "+v"(lim));   // one register, not a tile flag ANDed into every compare
      // dS as a bf16 pair (hi + lo): its rounding stays ~2^-16 relative.
      u32x4 dsh4[4], dsl4[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float pr[2], ds[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][r + e], c2, -lse2));
            if (32 * kb2 + 8 * ((r + e) >> 2) + ((r + e) & 3) > lim) pr[e] = 0.0f;
            if constexpr (DELTA) {
              dsum = __builtin_fmaf(pr[e], dp[kb2][r + e], dsum);
            } else {
              ds[e] = pr[e] * (dp[kb2][r + e] - dl);
            }
          }
          if constexpr (!DELTA) {
            unsigned hw, lw;
            split_pair(ds[0], ds[1], hw, lw);
            dsh4[2 * kb2 + (r >> 3)][(r & 7) >> 1] = hw;
            dsl4[2 * kb2 + (r >> 3)][(r & 7) >> 1] = lw;
          }
        }
      bf16x8 dsb[4], dsl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dsb[t] = __builtin_bit_cast(bf16x8, dsh4[t]);
        dsl[t] = __builtin_bit_cast(bf16x8, dsl4[t]);
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
    if (valid && half == 0) {
      p.delta[qrow_idx] = total;
      p.lse2[qrow_idx] = lse2;
    }
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
// One workgroup of 4 waves per (64-key tile, kv head); wave w owns keys
// 16w .. 16w+15 of the tile, so that its K and V operands and its dK, dV
// accumulators fit two waves per SIMD (whose vector and matrix work then
// overlap). Row blocks of 32 rows stream through a three-stage LDS ring.
constexpr int kDkvWaves = 4;
constexpr int kDkvKeysPerWave = 16;
constexpr int kRowsPerBlock = 32;

// 4-byte global -> LDS copy: lane i's 4 bytes land at lds + 4 * i.
__device__ __forceinline__ void load_lds4(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 4, 0, 0);
}

// Workgroup barrier for LDS only. __syncthreads() also waits for every vector
// memory operation in flight (its release fence covers the copies into LDS),
// which would drain the ring; the copies a stage needs are waited for
// explicitly with wait_vmcnt before this barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Chunk swizzle of the dK/dV kernel's row blocks. For 16 chunks per row it was
// chosen by timing both read patterns of this kernel on gfx950: 16 consecutive
// rows at one chunk per 16-lane group (operands of S and dP; two other XOR
// swizzles run these reads about 1.7 times slower) and the transposed reads of
// the dV and dK operands.
template <int CPR>
__device__ __forceinline__ int swz_kv(int r) {
  if constexpr (CPR == 16) {
    return ((r & 1) << 3) | ((r >> 1) & 7);
  } else {
    return (r >> 1) & 7;
  }
}

// Byte offset of the 8-byte piece (row, col .. col+3) in a row-major tile with
// ROWB-byte rows whose 16-byte chunks are swizzled by swz_kv<CPR>(row).
template <int CPR, int ROWB>
__device__ __forceinline__ int piece_kv(int row, int col) {
  return row * ROWB + (((col >> 3) ^ swz_kv<CPR>(row)) << 4) + ((col & 4) << 1);
}

template <int DQK, int DV>
struct DkvShape {
  static constexpr int KCPR = DQK / 8, VCPR = DV / 8;
  static constexpr int KROWB = DQK * 2, VROWB = DV * 2;
  static constexpr int QBYTES = kRowsPerBlock * KROWB, OBYTES = kRowsPerBlock * VROWB;
  // stage: Q block, dO block, then per-row lse2 and D
  static constexpr int INFO = QBYTES + OBYTES;
  static constexpr int STAGE = INFO + 2 * kRowsPerBlock * 4;
  static constexpr int Q_IPW = kRowsPerBlock * KCPR / 64 / kDkvWaves;   // copies per wave
  static constexpr int O_IPW = kRowsPerBlock * VCPR / 64 / kDkvWaves;
  static constexpr int LOADS = Q_IPW + O_IPW;   // waves 0 and 1 issue one row-info copy more
  static constexpr int KS = DQK / 32, VS = DV / 32;           // k-steps of S and dP
  static constexpr int KT = DQK / 16, VT = DV / 16;           // 16-wide tiles of dK and dV
  static_assert(kRowsPerBlock * KCPR % (64 * kDkvWaves) == 0, "Q block must split evenly");
  static_assert(kRowsPerBlock * VCPR % (64 * kDkvWaves) == 0, "dO block must split evenly");
};

// A block of 32 consecutive rows (token-major: all G heads of a kv head) of
// one query tile; t >= q_end marks the end of the walk.
struct RowBlock {
  int t, sb;    // query tile, block within it
  int qg;       // tile's first global position
  int nrg;      // tile's rows: tokens times G
  size_t base;  // index into [T_local * Hq] of the tile's first row
};

// Three workgroups per CU for d_qk <= 128 (at most 168 registers per lane,
// which the kernel fits without spilling): one wave's vector work then
// overlaps two others' MFMAs. The d_qk = 192 kernel needs more and runs two.
template <int DQK, int DV>
__global__ __launch_bounds__(kDkvWaves * 64, DQK > 128 ? 2 : 3) void thd_bwd_dkdv_kernel(BwdParams p) {
  using S = DkvShape<DQK, DV>;
  // Separate arrays, so the compiler can tell that reading one stage needs
  // no wait on copies still landing in another.
  __shared__ __attribute__((aligned(1024))) char stage0[S::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[S::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[S::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;   // 16-lane group
  const int lr = lane & 15;

  const int kvh = blockIdx.x % p.hkv;
  // Key tiles go out most-seen first (kv_order), so the longest walks start
  // first and the short ones fill in at the end.
  const int kt = ((const cint32_t*)p.kv_order)[blockIdx.x / p.hkv];
  // The tables are read-only for the whole launch: reading them through the
  // constant address space lets uniform reads use scalar loads.
  const cint32_t* kd = (const cint32_t*)(p.kvtiles) + size_t(kt) * 8;
  const int ks = kd[1], nk = kd[2], qb = kd[3], qe = kd[4];
  const int G = p.group;
  const int hkv = p.hkv;
  const int hq = p.hq;
  // floor(x / G) = (x * ginv) >> 16 for 0 <= x < 65536 / G; rows within a
  // tile number at most 128 and G at most 128.
  const uint32_t ginv = 65536u / uint32_t(G) + 1u;
  const uint32_t hq_minus_g = uint32_t(hq - G);
  const char* __restrict__ qbase = static_cast<const char*>(p.q);
  const char* __restrict__ obase = static_cast<const char*>(p.d_o);

  // This lane's key (lane % 16 of the wave's 16) as the B operand of S = Q K^T
  // and dP = dO V^T, held in registers for the whole walk. Keys past the
  // tile's end repeat its last key; their accumulators are never stored.
  const int key_rel = wave * kDkvKeysPerWave + lr;
  const int key = ks + key_rel;
  bf16x8 kf[S::KS], vf[S::VS];
  if (qb < qe) {
    const size_t kvr = size_t(p.kv_row[ks + min(key_rel, nk - 1)]) * hkv + kvh;
    const __bf16* krow = static_cast<const __bf16*>(p.k) + kvr * DQK + 8 * grp;
    const __bf16* vrow = static_cast<const __bf16*>(p.v) + kvr * DV + 8 * grp;
#pragma unroll
    for (int st = 0; st < S::KS; ++st) kf[st] = *reinterpret_cast<const bf16x8*>(krow + 32 * st);
#pragma unroll
    for (int st = 0; st < S::VS; ++st) vf[st] = *reinterpret_cast<const bf16x8*>(vrow + 32 * st);
    // Landed before the walk: pending at the loop's entry, these loads would
    // make the compiler wait for every copy in flight inside the loop.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  } else {
#pragma unroll
    for (int st = 0; st < S::KS; ++st) kf[st] = bf16x8{};
#pragma unroll
    for (int st = 0; st < S::VS; ++st) vf[st] = bf16x8{};
  }

  // Records (first local row, first position, rows) of the query tiles
  // [win, win + 64) that see this key tile, one tile per lane: the walk reads
  // them with readlane, without a memory round trip per tile.
  int win = qb, rec_ql = 0, rec_qg = 0, rec_nr = 0;
  auto load_window = [&](int w0) {
    win = w0;
    if (w0 + lane < qe) {
      const int32_t* td = p.tiles + size_t(w0 + lane) * 8;
      rec_ql = td[0];
      rec_qg = td[1];
      rec_nr = td[2];
    }
    // Resolved here, on this rare path: otherwise the compiler cannot tell
    // at the walk's merge points whether these loads are still in flight,
    // and waits for every copy in flight before each tile's readlanes.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };
  if (qb < qe) load_window(qb);
  auto load_tile = [&](int t) -> RowBlock {
    RowBlock b{t, 0, 0, 0, 0};
    if (t < qe) {
      if (t - win >= 64) load_window(t);
      const int idx = t - win;
      b.qg = __builtin_amdgcn_readlane(rec_qg, idx);
      b.nrg = __builtin_amdgcn_readlane(rec_nr, idx) * G;
      b.base = size_t(__builtin_amdgcn_readlane(rec_ql, idx)) * hq + kvh * G;
    }
    return b;
  };
  auto next_block = [&](const RowBlock& b) -> RowBlock {
    if (b.t >= qe) return b;
    if ((b.sb + 1) * kRowsPerBlock < b.nrg) return RowBlock{b.t, b.sb + 1, b.qg, b.nrg, b.base};
    return load_tile(b.t + 1);
  };
  // Row x of block b, as an offset from the tile's first row in [T_local * Hq]
  // (token * Hq + head in group). Rows past the tile's end repeat its last row
  // (the causal compare masks them out). Every factor is below 2^24.
  auto row_off = [&](const RowBlock& b, int x) -> uint32_t {
    const uint32_t rc = uint32_t(min(b.sb * kRowsPerBlock + x, b.nrg - 1)) & 127u;
    const uint32_t tok = (rc * (opaque(ginv) & 0x1ffffu)) >> 16;
    return rc + tok * (opaque(hq_minus_g) & 0xffffffu);   // tok * Hq + (rc - tok * G)
  };
  // When G divides 32, every block starts on a token, so in a block that lies
  // wholly inside its tile row r is token r / G, head r % G of the block's first
  // token: each lane's copy offsets are fixed for the whole walk and only a
  // scalar base moves from block to block.
  const bool aligned_blocks = kRowsPerBlock % G == 0;
  const int tokens_per_block = kRowsPerBlock / G;
  uint32_t qoff[S::Q_IPW], ooff[S::O_IPW];
#pragma unroll
  for (int i = 0; i < S::Q_IPW; ++i) {
    const int q = (wave * S::Q_IPW + i) * 64 + lane;
    const int r = q / S::KCPR;
    const int c = (q - r * S::KCPR) ^ swz_kv<S::KCPR>(r);
    qoff[i] = uint32_t(((r / G) * hq + r % G) * S::KROWB + c * 16);
  }
#pragma unroll
  for (int i = 0; i < S::O_IPW; ++i) {
    const int q = (wave * S::O_IPW + i) * 64 + lane;
    const int r = q / S::VCPR;
    const int c = (q - r * S::VCPR) ^ swz_kv<S::VCPR>(r);
    ooff[i] = uint32_t(((r / G) * hq + r % G) * S::VROWB + c * 16);
  }
  const uint32_t ioff = uint32_t((lane / G) * hq + lane % G);
  // Each wave issues S::LOADS copies per block, waves 0 and 1 one more (the
  // rows' lse2 and D).
  auto issue_block = [&](const RowBlock& b, char* stage) {
    const float* info = wave == 0 ? p.lse2 : p.delta;
    char* info_lds = stage + S::INFO + wave * kRowsPerBlock * 4;
    if (aligned_blocks && (b.sb + 1) * kRowsPerBlock <= b.nrg) {
      const size_t rb = b.base + size_t(b.sb * tokens_per_block) * hq;
      const char* qt = qbase + rb * S::KROWB;
      const char* ot = obase + rb * S::VROWB;
      // The offsets pass through an empty asm so that they stay 32-bit
      // registers: the compiler would otherwise keep 64-bit copies across the
      // walk and spill them at d_qk = 192 (every reload then waits for all
      // copies in flight).
#pragma unroll
      for (int i = 0; i < S::Q_IPW; ++i) {
        uint32_t off = qoff[i];
        asm volatile("" : "+v"(off));
        load_lds16(qt + off, stage + (wave * S::Q_IPW + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < S::O_IPW; ++i) {
        uint32_t off = ooff[i];
        asm volatile("" : "+v"(off));
        load_lds16(ot + off, stage + S::QBYTES + (wave * S::O_IPW + i) * 1024);
      }
      // gathered straight into LDS: a register load here would have to wait
      // for every copy issued before it
      if (wave < 2 && lane < kRowsPerBlock) load_lds4(reinterpret_cast<const char*>(info + rb + ioff), info_lds);
      return;
    }
    const char* qt = qbase + b.base * S::KROWB;
    const char* ot = obase + b.base * S::VROWB;
    // The lane's chunk offsets are recomputed from an opaque copy of the lane
    // id: kept live across the walk instead, they spill at d_qk = 192, and
    // every reload of a spill waits for all copies in flight.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < S::Q_IPW; ++i) {
      const int q = (wave * S::Q_IPW + i) * 64 + ln;
      const int r = q / S::KCPR;
      const int c = (q - r * S::KCPR) ^ swz_kv<S::KCPR>(r);
      load_lds16(qt + (row_off(b, r) * S::KROWB + c * 16), stage + (wave * S::Q_IPW + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < S::O_IPW; ++i) {
      const int q = (wave * S::O_IPW + i) * 64 + ln;
      const int r = q / S::VCPR;
      const int c = (q - r * S::VCPR) ^ swz_kv<S::VCPR>(r);
      load_lds16(ot + (row_off(b, r) * S::VROWB + c * 16), stage + S::QBYTES + (wave * S::O_IPW + i) * 1024);
    }
    if (wave < 2 && lane < kRowsPerBlock)
      load_lds4(reinterpret_cast<const char*>(info + b.base + row_off(b, lane)), info_lds);
  };
  auto wait_block = [&](bool one_in_flight) {
    if (!one_in_flight) {
      wait_vmcnt<0>();
    } else if (wave < 2) {
      wait_vmcnt<S::LOADS + 1>();
    } else {
      wait_vmcnt<S::LOADS>();
    }
  };

  f32x4 dk[S::KT], dv[S::VT];
#pragma unroll
  for (int b = 0; b < S::KT; ++b) dk[b] = f32x4{};
#pragma unroll
  for (int b = 0; b < S::VT; ++b) dv[b] = f32x4{};

  const float c2 = p.scale_log2;
  const int tr_row = 4 * grp + (lr >> 2);   // transposed reads: row within a 16-row half
  const int tr_col = 4 * (lr & 3);

  // One row block: S = Q K^T and dP = dO V^T (lane: key lane%16, rows
  // 16rt + 4*grp + i), P and dS as bf16 (hi, lo) pairs, then dV += P^T dO and
  // dK += dS^T Q with k-slot 8*grp + j of the pairs holding row
  // 16*(j/4) + 4*grp + j%4 and the B operands read transposed to match.
  auto compute = [&](const char* stage, const RowBlock& b) {
    f32x4 s[2] = {f32x4{}, f32x4{}}, dp[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 16 * rt + lr;
#pragma unroll
      for (int st = 0; st < (S::KS > S::VS ? S::KS : S::VS); ++st) {
        if (st < S::KS) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              stage + r * S::KROWB + (((4 * st + grp) ^ swz_kv<S::KCPR>(r)) << 4));
          s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[st], s[rt], 0, 0, 0);
        }
        if (st < S::VS) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              stage + S::QBYTES + r * S::VROWB + (((4 * st + grp) ^ swz_kv<S::VCPR>(r)) << 4));
          dp[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vf[st], dp[rt], 0, 0, 0);
        }
      }
    }
    // Rows of the block that see this lane's key: lo <= row < lo + span. Row
    // ri = sb*32 + row of the tile sits at position qg + floor(ri / G), which
    // is >= key exactly when ri >= (key - qg) * G; rows past the tile's rows
    // see nothing.
    const int kd_rel = min(max(key - b.qg, -1), 256);
    const int lo = max(kd_rel * int(opaque(uint32_t(G)) & 0xffu) - b.sb * kRowsPerBlock, 0);
    const int hi = min(b.nrg - b.sb * kRowsPerBlock, kRowsPerBlock);
    const uint32_t span = uint32_t(max(hi - lo, 0));
    const int row_bias = 4 * grp - lo;
    const float* info = reinterpret_cast<const float*>(stage + S::INFO);
    // Blocks whose every row sees every key of this wave (all 32 rows real,
    // the first row at or past the wave's last key) skip the per-element
    // test; the condition is wave-uniform. Keys past the tile's end only feed
    // accumulators that are never stored. The clamp keeps the product in
    // range and changes no outcome: a tile holds fewer than 256 tokens.
    const int key_hi = ks + wave * kDkvKeysPerWave + kDkvKeysPerWave - 1;
    const bool whole = b.nrg - b.sb * kRowsPerBlock >= kRowsPerBlock &&
                       min(max(key_hi - b.qg, -1), 256) * G <= b.sb * kRowsPerBlock;
    float pr[2][4], d4v[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r0 = 16 * rt + 4 * grp;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(info + r0);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(info + kRowsPerBlock + r0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[rt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][i], c2, -l4[i]));
        d4v[rt][i] = d4[i];
      }
    }
    if (!whole) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pr[rt][i] = uint32_t(16 * rt + i + row_bias) < span ? pr[rt][i] : 0.0f;
    }
    u32x4 ph, pl, dh, dl;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ds[i] = pr[rt][i] * (dp[rt][i] - d4v[rt][i]);
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        unsigned hw, lw;
        split_pair(pr[rt][i], pr[rt][i + 1], hw, lw);
        ph[2 * rt + i / 2] = hw;
        pl[2 * rt + i / 2] = lw;
        split_pair(ds[i], ds[i + 1], hw, lw);
        dh[2 * rt + i / 2] = hw;
        dl[2 * rt + i / 2] = lw;
      }
    }
    const bf16x8 pt = __builtin_bit_cast(bf16x8, ph), ptl = __builtin_bit_cast(bf16x8, pl);
    const bf16x8 dst = __builtin_bit_cast(bf16x8, dh), dsl = __builtin_bit_cast(bf16x8, dl);
#pragma unroll
    for (int nt = 0; nt < S::VT; ++nt) {
      const int col = 16 * nt + tr_col;
      const bf16x8 o8 = tr_pair(stage + S::QBYTES, piece_kv<S::VCPR, S::VROWB>(tr_row, col),
                                piece_kv<S::VCPR, S::VROWB>(16 + tr_row, col));
      dv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pt, o8, dv[nt], 0, 0, 0);
      dv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ptl, o8, dv[nt], 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < S::KT; ++nt) {
      const int col = 16 * nt + tr_col;
      const bf16x8 q8 = tr_pair(stage, piece_kv<S::KCPR, S::KROWB>(tr_row, col),
                                piece_kv<S::KCPR, S::KROWB>(16 + tr_row, col));
      dk[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dst, q8, dk[nt], 0, 0, 0);
      dk[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsl, q8, dk[nt], 0, 0, 0);
    }
  };

  if (qb < qe) {
    // Walk: block i is computed from stage i % 3 while block i + 1 lands and
    // block i + 2 is issued into the stage block i - 1 used.
    RowBlock b0 = load_tile(qb);
    RowBlock b1 = next_block(b0);
    RowBlock b2 = next_block(b1);
    issue_block(b0, stage0);
    if (b1.t < qe) issue_block(b1, stage1);
    wait_block(b1.t < qe);
    lds_barrier();
    auto step = [&](const char* cur, char* ahead) -> bool {
      if (b0.t >= qe) return false;
      const bool have2 = b2.t < qe;
      if (have2) issue_block(b2, ahead);
      const RowBlock b3 = next_block(b2);
      compute(cur, b0);
      wait_block(have2);
      lds_barrier();
      b0 = b1;
      b1 = b2;
      b2 = b3;
      return true;
    };
    while (step(stage0, stage2) && step(stage1, stage0) && step(stage2, stage1)) {
    }
  }

  // Store: lane holds dims 16nt + lane%16 of keys 16*wave + 4*grp + i.
  // All row indices are read before the first store (a store could alias them).
  int grows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = wave * kDkvKeysPerWave + 4 * grp + i;
    grows[i] = kr < nk ? p.kv_row[ks + kr] : -1;
  }
  // bf16 output: the same fp32 values, rounded to nearest even.
  const bool out_bf16 = p.kv_bf16 != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (grows[i] < 0) continue;
    const size_t grow = size_t(grows[i]) * hkv + kvh;
    if (out_bf16) {
      __bf16* dk16 = static_cast<__bf16*>(p.dk) + grow * DQK + lr;
      __bf16* dv16 = static_cast<__bf16*>(p.dv) + grow * DV + lr;
#pragma unroll
      for (int nt = 0; nt < S::KT; ++nt) dk16[16 * nt] = static_cast<__bf16>(dk[nt][i] * p.scale);
#pragma unroll
      for (int nt = 0; nt < S::VT; ++nt) dv16[16 * nt] = static_cast<__bf16>(dv[nt][i]);
    } else {
      float* dk32 = static_cast<float*>(p.dk) + grow * DQK + lr;
      float* dv32 = static_cast<float*>(p.dv) + grow * DV + lr;
#pragma unroll
      for (int nt = 0; nt < S::KT; ++nt) dk32[16 * nt] = dk[nt][i] * p.scale;
#pragma unroll
      for (int nt = 0; nt < S::VT; ++nt) dv32[16 * nt] = dv[nt][i];
    }
  }
}

template <int DQK, int DV>
int launch(const BwdParams& p, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 q_grid(unsigned(int64_t(p.n_tiles) * p.hkv));
  const dim3 kv_grid(unsigned(int64_t(p.n_kvtiles) * p.hkv));
  hipError_t err;
  if (p.o_f32 != nullptr) {
    // dQ first: it computes D from the exact O and stores D and lse2.
    hipLaunchKernelGGL((thd_bwd_dq_kernel<DQK, DV, false>), q_grid, dim3(kWaves * 64), 0, st, p);
    err = hipGetLastError();
    if (err != hipSuccess) return int(err);
    hipLaunchKernelGGL((thd_bwd_dkdv_kernel<DQK, DV>), kv_grid, dim3(kDkvWaves * 64), 0, st, p);
    return int(hipGetLastError());
  }
  hipLaunchKernelGGL((thd_bwd_dq_kernel<DQK, DV, true>), q_grid, dim3(kWaves * 64), 0, st, p);
  err = hipGetLastError();
  if (err != hipSuccess) return int(err);
  hipLaunchKernelGGL((thd_bwd_dkdv_kernel<DQK, DV>), kv_grid, dim3(kDkvWaves * 64), 0, st, p);
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
