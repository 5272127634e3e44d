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
#include <type_traits>

#include "ffa_internal.hpp"

namespace ffa {

namespace {

constexpr int NT = 256;

template <int D>
__global__ __launch_bounds__(NT, 2) void ffa_fwd_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILE_B = BN_F * D * 2;          // bytes of one K or V tile
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int KB = BN_F / 32;                 // 32-key blocks per tile
  constexpr int MB = D / 32;                    // 32-wide d blocks of O^T
  constexpr int KS = D / 16;                    // 16-wide d steps of S^T

  const MetaView mv = meta_view(a.meta);
  const FFA_CONST MetaHeader* hd = mv.hdr;
  if (hd->status != 0 || hd->seqlen_q != a.Tq || hd->seqlen_k != a.Tk) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31, h32 = lane >> 5, t16 = lane & 15, g16 = lane >> 4;
  const int head = blockIdx.x % a.Hq;
  const int m = mv.sched_f[blockIdx.x / a.Hq];
  const int kvh = head / (a.Hq / a.Hkv);
  const int qrow = m * BM_F + wid * 32 + l32;
  const bool qok = qrow < a.Tq;

  const int f0 = mv.qf_off[m], nF = mv.qf_off[m + 1] - f0;
  const int p0 = mv.qm_off[m], nP = mv.qm_off[m + 1] - p0;
  const int nT = nP + nF;
  cint32_t* fidx = mv.var + hd->list_off[L_QF] + f0;
  cint32_t* pidx = mv.var + hd->list_off[L_QM] + p0;
  const int s0 = mv.qs_off[m], nS = mv.qs_off[m + 1] - s0;
  cint32_t* sidx = mv.var + hd->list_off[L_QS] + s0;

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

  wait_vmem();

  // loop-invariant LDS read bases (stage, key block, column group and chunk
  // offsets are immediates): the 128-bit K read of chunk 2k + h32 is at
  // (k / 2) * GB + kaddr[k % 2], the transposed V read of rows 8j.. of column
  // group mb at mb * GB + vaddr[j]
  constexpr int GB = group_bytes<BN_F>();
  int kaddr[2], vaddr[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) kaddr[p] = lds_pos(l32, 2 * p + h32);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    vaddr[j] = lds_pos(4 * h32 + (t16 >> 2) + 8 * j, 2 * (g16 & 1) + ((t16 >> 1) & 1)) + 8 * (t16 & 1);

  TileDma<D, BN_F> dma;
  dma.init(wid, lane, a.k_ts);
  TileDma<D, BN_F> dmv;
  dmv.init(wid, lane, a.v_ts);
  const __bf16* kbase = a.k + (int64_t)kvh * a.k_hs;
  const __bf16* vbase = a.v + (int64_t)kvh * a.v_hs;
  auto tile_of = [&](int t) { return t < nP ? pidx[t] : fidx[t - nP]; };
  auto issue = [&](int t, int stage) {
    const int n = tile_of(t);
    char* st = smem + stage * STAGE_B;
    dma.load(kbase, a.k_ts, n * BN_F, a.Tk - n * BN_F, st);
    dmv.load(vbase, a.v_ts, n * BN_F, a.Tk - n * BN_F, st + TILE_B);
  };

  f32x16 oacc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;   // running max of raw scores, partial row sum
  const float c = a.scale_log2;           // > 0
  const float thr = 8.f / c;              // rescale only when the max grows by 2^8

  auto tile = [&](auto stage_c, int t) {
    constexpr int stage = decltype(stage_c)::value;
    const bool masked = t < nP;
    const int n = tile_of(t);
    if (t + 1 < nT) issue(t + 1, stage ^ 1);
    const __attribute__((address_space(3))) char* lb =
        (const __attribute__((address_space(3))) char*)smem + stage * STAGE_B;

    // S^T = K Q^T; two independent accumulation chains interleaved
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4 u = *(const __attribute__((address_space(3))) u32x4*)(lb + (k >> 1) * GB + kaddr[k & 1] + kb * 32 * 64);
        bf16x8 kop;
        __builtin_memcpy(&kop, &u, 16);
        sacc[kb] = mfma32(kop, qop[k], sacc[kb]);
      }

    if (masked) {
      const int n0 = n * BN_F;
      uint64_t mk = 0;
      for (int si = 0; si < nS; ++si) {
        const Slice sl = load_slice(mv.slices, sidx[si]);
        int lo, hi;
        row_interval(sl, qrow, lo, hi);
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
          if (!((w >> (8 * (r >> 2) + (r & 3))) & 1u)) sacc[kb][r] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = wave_swap_max(mx);
    if (__ballot(mx > m_run + thr) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, -mc));
        sacc[kb][r] = pv;
        psum += pv;
      }
    l_run += psum;

    // O^T += V^T P^T over 16-key chunks
#pragma unroll
    for (int cc = 0; cc < BN_F / 16; ++cc) {
      const int kb = cc >> 1, c2 = cc & 1;
      bf16x8 pop;
#pragma unroll
      for (int e = 0; e < 8; ++e) pop[e] = static_cast<__bf16>(sacc[kb][8 * c2 + e]);
      const int roff = TILE_B + (32 * kb + 16 * c2) * 64;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(lb + mb * GB + vaddr[0] + roff));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(lb + mb * GB + vaddr[1] + roff));
        const i16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 vop;
        __builtin_memcpy(&vop, &vv, 16);
        oacc[mb] = mfma32(vop, pop, oacc[mb]);
      }
    }
    wait_dma();
    __syncthreads();
  };

  if (nT > 0) issue(0, 0);
  wait_dma();
  __syncthreads();
  for (int t = 0; t < nT; t += 2) {
    tile(std::integral_constant<int, 0>{}, t);
    if (t + 1 < nT) tile(std::integral_constant<int, 1>{}, t + 1);
  }

  // epilogue: O = O^T / l, LSE = m*scale + ln l (natural log)
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
      a.lse[(int64_t)head * a.Tq + qrow] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
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
