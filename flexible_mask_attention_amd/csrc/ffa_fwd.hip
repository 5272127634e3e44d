// ffa_fwd.hip - Flex-Flash-Attention forward on gfx950.
//
// Fused S = scale * Q K^T -> masked online softmax -> O = P V over the q2k
// Full and Partial key tiles of each query block, the FFA kernel's job on the
// MagiAttention pages (blog deep-dive, section "Flex-Flash-Attention 与
// AttnSlice", Fig. 5: data loading plus on-chip compute per slice), with the
// create_block_mask / CSR tile lists of the documentation page ("FFA_FA4"
// optimisations) so that only Partial tiles pay for per-element masking.
//
// Work item: (query head, 128-row query block), 4 waves, 32 query rows each.
// The kernel computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that each
// lane owns one query row: its softmax statistics stay in registers and only
// one half-wave swap is needed per row max.  The P^T accumulator registers
// feed the next MFMA (O^T += V^T P^T) directly as its B operand; V^T comes
// from LDS through ds_read_b64_tr_b16.  K and V tiles are double-buffered in
// LDS; global loads for tile t+1 are issued before tile t is computed.
#include "ffa_internal.hpp"

namespace ffa {

namespace {

constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT, 2) void ffa_fwd_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILE_B = BN_F * D * 2;          // bytes of one K or V tile
  constexpr int NCH = D / 8;                    // 16-byte chunks per row
  constexpr int PERT = BN_F * NCH / NT;         // chunks per thread per tile
  constexpr int KB = BN_F / 32;                 // 32-key blocks per tile
  constexpr int MB = D / 32;                    // 32-wide d blocks of O^T
  constexpr int KS = D / 16;                    // 16-wide d steps of S^T

  const MetaView mv = meta_view(a.meta);
  const MetaHeader* hd = mv.hdr;
  if (hd->status != 0 || hd->seqlen_q != a.Tq || hd->seqlen_k != a.Tk) return;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h32 = lane >> 5, t16 = lane & 15, g16 = lane >> 4;
  const int head = blockIdx.x % a.Hq;
  const int m = mv.sched_f[blockIdx.x / a.Hq];
  const int kvh = head / (a.Hq / a.Hkv);
  const int qrow = m * BM_F + wid * 32 + l32;
  const bool qok = qrow < a.Tq;

  const int f0 = mv.qf_off[m], nF = mv.qf_off[m + 1] - f0;
  const int p0 = mv.qm_off[m], nP = mv.qm_off[m + 1] - p0;
  const int nT = nP + nF;
  const int32_t* fidx = mv.var + hd->list_off[L_QF] + f0;
  const int32_t* pidx = mv.var + hd->list_off[L_QM] + p0;
  const int s0 = mv.qs_off[m], nS = mv.qs_off[m + 1] - s0;
  const int32_t* sidx = mv.var + hd->list_off[L_QS] + s0;

  // Q^T operand: lane holds Q[qrow][16k + 8*h32 + e]
  bf16x8 qop[KS];
  {
    const __bf16* qp = a.q + (int64_t)qrow * a.q_ts + (int64_t)head * a.q_hs + 8 * h32;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u32x4 u = qok ? *reinterpret_cast<const u32x4*>(qp + 16 * k) : u32x4{0, 0, 0, 0};
      __builtin_memcpy(&qop[k], &u, 16);
    }
  }

  f32x16 oacc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const __bf16* kbase = a.k + (int64_t)kvh * a.k_hs;
  const __bf16* vbase = a.v + (int64_t)kvh * a.v_hs;
  u32x4 kreg[PERT], vreg[PERT];
  auto tile_of = [&](int t) { return t < nP ? pidx[t] : fidx[t - nP]; };
  auto gload = [&](int n) {
#pragma unroll
    for (int i = 0; i < PERT; ++i) {
      const int idx = tid + NT * i, r = idx / NCH, c = idx % NCH;
      const int key = n * BN_F + r;
      if (key < a.Tk) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * a.k_ts + 8 * c);
        vreg[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * a.v_ts + 8 * c);
      } else {
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int stage) {
    char* kt = smem + stage * 2 * TILE_B;
    char* vt = kt + TILE_B;
#pragma unroll
    for (int i = 0; i < PERT; ++i) {
      const int idx = tid + NT * i, r = idx / NCH, c = idx % NCH;
      *reinterpret_cast<u32x4*>(kt + lds_off<D>(r, c)) = kreg[i];
      *reinterpret_cast<u32x4*>(vt + lds_off<D>(r, c)) = vreg[i];
    }
  };

  if (nT > 0) {
    gload(tile_of(0));
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < nT; ++t) {
    const int stage = t & 1;
    const bool masked = t < nP;
    const int n = tile_of(t);
    if (t + 1 < nT) gload(tile_of(t + 1));
    const char* kt = smem + stage * 2 * TILE_B;
    const char* vt = kt + TILE_B;

    // S^T = K Q^T: rows = keys 32kb + (8(r/4) + 4*h32 + r%4), column = this lane's query
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8 kop = read_row_operand<D>(kt, 32 * kb + l32, 2 * k + h32);
        sacc[kb] = mfma32(kop, qop[k], sacc[kb]);
      }
    }

    float x[KB][16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kb][r] = sacc[kb][r] * a.scale_log2;

    if (masked) {
      // valid keys of this row inside [n0, n0 + BN_F) as a bit mask
      const int n0 = n * BN_F;
      uint64_t mk = 0;
      for (int si = 0; si < nS; ++si) {
        const Slice s = load_slice(mv.slices, sidx[si]);
        int lo, hi;
        row_interval(s, qrow, lo, hi);
        lo = max(lo, n0);
        hi = min(hi, n0 + BN_F - 1);
        if (lo <= hi) mk |= bit_range(lo - n0, hi - n0);
      }
      mk >>= 4 * h32;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t w = static_cast<uint32_t>(mk >> (32 * kb));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) x[kb][r] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[kb][r]);
    mx = wave_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(x[kb][r] - m_use);
        x[kb][r] = pv;
        psum += pv;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;

    // O^T += V^T P^T over 16-key chunks
#pragma unroll
    for (int c = 0; c < BN_F / 16; ++c) {
      const int kb = c >> 1, c2 = c & 1;
      const bf16x8 pop = pack_bf16x8(&x[kb][8 * c2]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 vop = read_tr_operand<D>(vt, 32 * kb + 16 * c2 + 4 * h32,
                                              32 * mb + 16 * (g16 & 1), t16);
        oacc[mb] = mfma32(vop, pop, oacc[mb]);
      }
    }

    if (t + 1 < nT) lstore(stage ^ 1);
    __syncthreads();
  }

  // epilogue: O = O^T / l, LSE = m*ln2 + ln l (natural log, scale included)
  const float l_tot = wave_swap_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qok) {
    __bf16* op = a.o + (int64_t)qrow * a.o_ts + (int64_t)head * a.o_hs;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = static_cast<__bf16>(oacc[mb][4 * j + i] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * j + 4 * h32) = w;
      }
    if (h32 == 0)
      a.lse[(int64_t)head * a.Tq + qrow] = l_tot > 0.f ? m_run * LN2 + logf(l_tot) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int nq_f, hipStream_t stream) {
  const int64_t grid = (int64_t)nq_f * a.Hq;
  if (grid == 0) return hipSuccess;
  if (head_dim == 128) {
    const size_t lds = 2 * 2 * BN_F * 128 * 2;
    ffa_fwd_kernel<128><<<dim3((unsigned)grid), NT, lds, stream>>>(a);
  } else {
    const size_t lds = 2 * 2 * BN_F * 64 * 2;
    ffa_fwd_kernel<64><<<dim3((unsigned)grid), NT, lds, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ffa
