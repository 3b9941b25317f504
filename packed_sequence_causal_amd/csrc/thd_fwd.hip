// Forward kernel: causal + EOD-reset attention for one rank's query tiles
// against rank-major gathered K/V (gfx950, bf16 MFMA, fp32 accumulate).
//
// The operation is the one of "kvallgather cp thd load balance" (Ascend/
// MindSpeed, "What this PR does / why we need it?": THD attention with direct
// rank-major K/V indexing in a single fused call; "Does this PR introduce any
// user-facing change?": causal attention with the mask reset at every EOD).
//
// Work decomposition. One workgroup (4 waves, 256 lanes) handles one query
// tile of one kv head: block_t tokens x G q heads = up to 128 rows, token-major
// (row = token * G + head-in-group), 32 rows per wave. All G heads of a kv head
// share every K/V tile, so a K/V tile loaded once into LDS feeds 128 rows even
// when tiles hold few tokens. Workgroup b takes kv head b % Hkv and tile
// order[b / Hkv]: tiles are dispatched longest first, and since workgroups are
// spread round robin over the 8 XCDs, with Hkv = 8 each XCD (and its L2) serves
// a single kv head.
//
// Per KV tile of 64 keys (only the tiles from the document start up to the
// tile's last row are visited):
//   * the next tile's K rows and V rows are fetched with 16-byte global loads
//     into registers while the current tile is computed; the row of each key
//     comes from the gathered-row map (no reorder copy of K/V);
//   * K is stored to LDS row-major, V transposed (V^T), so both MFMA operands
//     read contiguous runs along the contraction dimension;
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
//     of P^T, so P never leaves registers.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "internal.h"

namespace thd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = kWaves * 64;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;

template <int DQK, int DV>
struct FwdShape {
  static constexpr int BN = kBlockN;
  static constexpr int KLD = DQK + 8;        // LDS K row stride (bf16), 16-byte pad
  static constexpr int VLD = BN + 4;         // LDS V^T row stride (bf16), 8-byte pad
  static constexpr int KCH = DQK / 8;        // 16-byte chunks per K row
  static constexpr int K_LOADS = BN * KCH / kThreads;
  static constexpr int V_CH = DV / 8;        // 16-byte chunks per V row
  static constexpr int V_BLOCKS = (BN / 4) * V_CH;   // 4 keys x 8 dims each
  static constexpr int V_LOADS = (V_BLOCKS + kThreads - 1) / kThreads;
  static constexpr int KSTEPS = DQK / 16;
  static constexpr int DVB = DV / 32;
  static_assert(BN * KCH % kThreads == 0, "K tile must split evenly over the workgroup");
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims must suit the MFMA tiles");
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);   // a.lo16 | b.lo16 << 16
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);   // a.hi16 | b.hi16 << 16
}

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void thd_fwd_kernel(FwdParams p) {
  using S = FwdShape<DQK, DV>;
  constexpr int BN = S::BN;
  __shared__ __attribute__((aligned(16))) __bf16 ks[BN * S::KLD];
  __shared__ __attribute__((aligned(16))) __bf16 vt[DV * S::VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;        // which 32-lane half
  const int lrow = lane & 31;

  const int kvh = blockIdx.x % p.hkv;
  const int tile = p.order[blockIdx.x / p.hkv];
  const int32_t* td = p.tiles + size_t(tile) * 8;
  const int q_local0 = td[0];
  const int q_glob0 = td[1];
  const int n_rows = td[2];
  const int kv_start = td[5];
  const int n_kv = td[6];
  const int n_full = td[7];
  const int key_end = q_glob0 + n_rows;    // keys from here on are seen by no row

  const int G = p.group;
  const int row = wave * 32 + lrow;
  const int tok = row / G;
  const int head = kvh * G + (row - tok * G);
  const bool valid = tok < n_rows;
  const int qpos = valid ? q_glob0 + tok : INT_MAX;
  const bool wave_active = (wave * 32) / G < n_rows;

  const __bf16* __restrict__ qp = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kp = static_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(p.v);
  const int hkv = p.hkv;

  // Q^T operand: lane holds Q[row][16*st + 8*half .. +7] for each k-step.
  bf16x8 qf[S::KSTEPS];
  {
    const __bf16* qrow = qp + (size_t(q_local0 + tok) * p.hq + head) * DQK + 8 * half;
#pragma unroll
    for (int st = 0; st < S::KSTEPS; ++st) {
      if (valid) {
        qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st);
      } else {
        qf[st] = bf16x8{};
      }
    }
  }

  uint4 kreg[S::K_LOADS];
  uint4 vreg[S::V_LOADS][4];

  auto fetch = [&](int j) {
    const int key0 = kv_start + j * BN;
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / S::KCH;
      const int col = c - r * S::KCH;
      const int key = key0 + r;
      if (key < key_end) {
        const int grow = p.kv_row[key];
        kreg[i] = *reinterpret_cast<const uint4*>(kp + (size_t(grow) * hkv + kvh) * DQK + col * 8);
      } else {
        kreg[i] = uint4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) {
      const int blk = tid + kThreads * i;
      const int dch = blk % S::V_CH;
      const int quad = blk / S::V_CH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + 4 * quad + e;
        if (blk < S::V_BLOCKS && key < key_end) {
          const int grow = p.kv_row[key];
          vreg[i][e] = *reinterpret_cast<const uint4*>(vp + (size_t(grow) * hkv + kvh) * DV + dch * 8);
        } else {
          vreg[i][e] = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < S::K_LOADS; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / S::KCH;
      const int col = c - r * S::KCH;
      *reinterpret_cast<uint4*>(&ks[r * S::KLD + col * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < S::V_LOADS; ++i) {
      const int blk = tid + kThreads * i;
      if (blk < S::V_BLOCKS) {
        const int dch = blk % S::V_CH;
        const int quad = blk / S::V_CH;
        const uint32_t w[4][4] = {{vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w},
                                  {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w},
                                  {vreg[i][2].x, vreg[i][2].y, vreg[i][2].z, vreg[i][2].w},
                                  {vreg[i][3].x, vreg[i][3].y, vreg[i][3].z, vreg[i][3].w}};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // dims 2m and 2m+1 of the four keys, as 4 consecutive bf16 each
          const uint2 even{lo_pair(w[0][m], w[1][m]), lo_pair(w[2][m], w[3][m])};
          const uint2 odd{hi_pair(w[0][m], w[1][m]), hi_pair(w[2][m], w[3][m])};
          const int d = dch * 8 + 2 * m;
          *reinterpret_cast<uint2*>(&vt[d * S::VLD + 4 * quad]) = even;
          *reinterpret_cast<uint2*>(&vt[(d + 1) * S::VLD + 4 * quad]) = odd;
        }
      }
    }
  };

  f32x16 acc[S::DVB];
#pragma unroll
  for (int b = 0; b < S::DVB; ++b) acc[b] = f32x16{};
  float m_run = -INFINITY;   // running max of scale*log2(e)*s for this lane's row
  float l_run = 0.0f;        // this lane's share of the row's sum of 2^(...)
  const float c2 = p.scale_log2;

  fetch(0);
  for (int j = 0; j < n_kv; ++j) {
    if (j > 0) __syncthreads();
    stash();
    __syncthreads();
    if (j + 1 < n_kv) fetch(j + 1);
    if (!wave_active) continue;

    // S^T = K Q^T for keys [32*kb, 32*kb + 32) of the tile.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int st = 0; st < S::KSTEPS; ++st) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ks[(32 * kb + lrow) * S::KLD + 16 * st + 8 * half]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
    }

    if (j >= n_full) {
      const int key0 = kv_start + j * BN + 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + (r & 3);
          if (key > qpos) s[kb][r] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Each row decides on its own (so a row's arithmetic never depends on
    // its neighbours); the wave only skips the rescale when no row needs it.
    const float m_tile = mx * c2;
    const bool need = m_tile > m_run + kRescaleSlack;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;
#pragma unroll
      for (int b = 0; b < S::DVB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
      l_run *= alpha;
      m_run = need ? m_tile : m_run;
    }

    const float neg_m = -m_run;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, neg_m));
        l_run += e;
        pb[2 * kb + (r >> 3)][r & 7] = static_cast<__bf16>(e);
      }

    // O^T += V^T P^T, 16 keys per MFMA: keys 16t + 4*half + {0..3, 8..11}.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int b = 0; b < S::DVB; ++b) {
        const __bf16* src = &vt[(32 * b + lrow) * S::VLD + 16 * t + 4 * half];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(src);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(src + 8);
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], acc[b], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!valid) return;
  const float inv = 1.0f / l_tot;
  __bf16* orow = static_cast<__bf16*>(p.o) + (size_t(q_local0 + tok) * p.hq + head) * DV;
#pragma unroll
  for (int b = 0; b < S::DVB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = static_cast<__bf16>(acc[b][4 * g + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * g + 4 * half) = out;
    }
  if (half == 0) p.lse[size_t(q_local0 + tok) * p.hq + head] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <int DQK, int DV>
int launch(const FwdParams& p, void* stream) {
  const dim3 grid(unsigned(int64_t(p.n_tiles) * p.hkv));
  hipLaunchKernelGGL((thd_fwd_kernel<DQK, DV>), grid, dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  return int(hipGetLastError());
}

}  // namespace

bool fwd_supported(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

int launch_fwd(const FwdParams& p, int d_qk, int d_v, void* stream) {
  if (d_qk == 64 && d_v == 64) return launch<64, 64>(p, stream);
  if (d_qk == 128 && d_v == 128) return launch<128, 128>(p, stream);
  if (d_qk == 192 && d_v == 128) return launch<192, 128>(p, stream);
  return int(hipErrorInvalidValue);
}

}  // namespace thd
