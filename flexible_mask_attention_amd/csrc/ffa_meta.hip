// ffa_meta.hip - block metadata of a slice table on gfx950.
//
// For every tile (query block x key block) the exact number v of valid
// (query, key) pairs is counted and the tile is classed Empty (v = 0), Full
// (no masking needed) or Partial (masking needed); the non-empty tiles of each
// block are listed in CSR form, Full and Partial apart.  This follows the
// create_block_mask kernel and CSR compression of the MagiAttention
// documentation page, "FFA_FA4" optimisations, items 1 and 2 (q2k for the
// forward, k2q for the backward, out-of-bounds-in-q-only blocks count as Full
// in the forward), rebuilt for AttnSlice tables:
//
//   q2k: owner = query block of BM_F rows, iterated = key blocks of BN_F.
//        Rows past seqlen_q are ignored; keys past seqlen_k are invalid.
//        Full iff v == rows_in_bounds * BN_F.
//   k2q: owner = key block of BN_B keys, iterated = query blocks of BM_B.
//        Keys past seqlen_k are ignored; rows past seqlen_q are invalid.
//        Full iff v == keys_in_bounds * BM_B.
//
// Counting: each owner position (a row for q2k, a key for k2q) has one valid
// interval per slice along the iterated axis.  An interval adds its length
// clipped to the two end blocks directly, and whole blocks in between through
// a difference array; a prefix sum then gives v for every iterated block.
// All integer work, so the result is exact and order independent.
#include "ffa_internal.hpp"

namespace ffa {

namespace {

constexpr int MT = 256;     // threads of the tile kernels
constexpr int CH = 4096;    // iterated blocks per LDS chunk
constexpr int PER = CH / MT;
// owners past MAX_SORT keep their natural order in the schedules
constexpr int MAX_SORT = 32768;

struct MetaPtrs {
  MetaHeader* hdr;
  int32_t* slices;
  int32_t* qf_off;
  int32_t* qm_off;
  int32_t* kf_off;
  int32_t* km_off;
  int32_t* qs_off;
  int32_t* sched_f;
  int32_t* sched_b;
  int32_t* rec_f;
  int32_t* rec_b;
  int32_t* var;
};

__device__ MetaPtrs meta_ptrs(void* meta) {
  char* b = reinterpret_cast<char*>(meta);
  MetaPtrs p;
  p.hdr = reinterpret_cast<MetaHeader*>(b);
  p.slices = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_SLICES]);
  p.qf_off = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_QF_OFF]);
  p.qm_off = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_QM_OFF]);
  p.kf_off = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_KF_OFF]);
  p.km_off = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_KM_OFF]);
  p.qs_off = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_QS_OFF]);
  p.sched_f = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_SCHED_F]);
  p.sched_b = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_SCHED_B]);
  p.rec_f = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_REC_F]);
  p.rec_b = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_REC_B]);
  p.var = reinterpret_cast<int32_t*>(b + p.hdr->byte_off[A_VAR]);
  return p;
}

struct InitArgs {
  int32_t S, Tq, Tk, head_dim;
  int32_t nq_f, nk_f, nq_b, nk_b;
  int64_t capacity;
  int64_t byte_off[11];
};

// Header fields, counters, and a copy of the slice table.
__global__ void meta_init_kernel(const int32_t* __restrict__ slices, void* meta, InitArgs a) {
  char* b = reinterpret_cast<char*>(meta);
  MetaHeader* h = reinterpret_cast<MetaHeader*>(b);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    h->magic = META_MAGIC;
    h->version = META_VERSION;
    h->status = 0;
    h->num_slices = a.S;
    h->seqlen_q = a.Tq;
    h->seqlen_k = a.Tk;
    h->head_dim = a.head_dim;
    h->pad0 = 0;
    h->bm_f = BM_F;
    h->bn_f = BN_F;
    h->bm_b = BM_B;
    h->bn_b = BN_B;
    h->nq_f = a.nq_f;
    h->nk_f = a.nk_f;
    h->nq_b = a.nq_b;
    h->nk_b = a.nk_b;
    h->capacity = a.capacity;
    h->area = 0;
    for (int i = 0; i < 5; ++i) {
      h->nnz[i] = 0;
      h->list_off[i] = 0;
    }
    for (int i = 0; i < 11; ++i) h->byte_off[i] = a.byte_off[i];
  }
  int32_t* dst = reinterpret_cast<int32_t*>(b + a.byte_off[A_SLICES]);
  const int n = 5 * a.S;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    dst[i] = slices[i];
}

// Per-slice bounds and type checks, one thread per slice.
__device__ void check_slices(void* meta, int blk) {
  MetaPtrs p = meta_ptrs(meta);
  const int S = p.hdr->num_slices, Tq = p.hdr->seqlen_q, Tk = p.hdr->seqlen_k;
  const int a = blk * MT + threadIdx.x;
  if (a >= S) return;
  const Slice s = load_slice(p.slices, a);
  const bool bounds = 0 <= s.q0 && s.q0 <= s.q1 && s.q1 <= Tq && 0 <= s.k0 && s.k0 <= s.k1 && s.k1 <= Tk;
  int flags = 0;
  if (!bounds) flags |= FFA_META_ERR_BOUNDS;
  else if (s.t < 0 || s.t > 3) flags |= FFA_META_ERR_TYPE;
  if (flags) atomicOr(&p.hdr->status, flags);
}

// A slice's valid keys in row i are [lo(i), hi(i)] with both ends linear in i
// (slope 1 where the mask type bounds that side by the diagonal, else 0), on
// the rows [A, B] where that interval is not empty (see row_interval: inside
// the slice's rows the causal bound never exceeds Lk - 1).
struct RowLines {
  int64_t A, B, lc, hc;
  int ls, hs;
};

__device__ RowLines row_lines(const Slice& s) {
  const int64_t Lq = s.q1 - s.q0, Lk = s.k1 - s.k0, D = Lk - Lq;
  const bool inv = (s.t == FFA_INV_CAUSAL) | (s.t == FFA_BI_CAUSAL);
  const bool cau = (s.t == FFA_CAUSAL) | (s.t == FFA_BI_CAUSAL);
  RowLines r;
  r.A = s.q0;
  r.B = static_cast<int64_t>(s.q1) - 1;
  if (cau) r.A = max(r.A, static_cast<int64_t>(s.q0) - D);     // r + D >= 0
  if (inv) r.B = min(r.B, static_cast<int64_t>(s.q0) + Lk - 1);  // r <= Lk - 1
  if (Lk <= 0 || (inv && cau && D < 0)) r.B = r.A - 1;            // no valid pair
  r.ls = inv ? 1 : 0;
  r.lc = inv ? static_cast<int64_t>(s.k0) - s.q0 : s.k0;
  r.hs = cau ? 1 : 0;
  r.hc = cau ? static_cast<int64_t>(s.k0) - s.q0 + D : static_cast<int64_t>(s.k0) + Lk - 1;
  return r;
}

// Do two slices share a valid (query, key) pair?  On their common valid rows
// [R0, R1], g(i) = min(hi_a, hi_b) - max(lo_a, lo_b) is concave and piecewise
// linear (a minimum of lines minus a maximum of lines), so its largest value
// is taken at R0, R1 or a row where two lines of different slope cross; those
// crossings are integers because the slopes differ by exactly 1.  The pair
// overlaps iff g >= 0 at one of these at most four rows.
__device__ bool pair_overlaps(const Slice& sa, const Slice& sb) {
  const RowLines x = row_lines(sa), y = row_lines(sb);
  const int64_t R0 = max(x.A, y.A), R1 = min(x.B, y.B);
  if (R0 > R1) return false;
  auto meets = [&](int64_t i) {
    const int64_t hi = min(x.hc + x.hs * i, y.hc + y.hs * i);
    const int64_t lo = max(x.lc + x.ls * i, y.lc + y.ls * i);
    return hi >= lo;
  };
  if (meets(R0) || meets(R1)) return true;
  if (x.hs != y.hs) {
    const int64_t c = (y.hc - x.hc) / (x.hs - y.hs);
    if (c > R0 && c < R1 && meets(c)) return true;
  }
  if (x.ls != y.ls) {
    const int64_t c = (y.lc - x.lc) / (x.ls - y.ls);
    if (c > R0 && c < R1 && meets(c)) return true;
  }
  return false;
}

// Disjointness, tested in the query block where two slices' common rows
// begin: both are on that block's slice list, and every pair of slices with
// common rows is tested by exactly one block.  The cost is the sum over query
// blocks of (slices meeting the block)^2 / 2, so a table whose rows each meet
// a bounded number of slices is checked in time linear in its size.
__device__ void validate_pairs(MetaPtrs p, const int32_t* list, int k, int a0, int a1) {
  for (int x = 0; x + 1 < k; ++x) {
    const Slice sa = load_slice(p.slices, list[x]);
    for (int y = x + 1 + static_cast<int>(threadIdx.x); y < k; y += MT) {
      const Slice sb = load_slice(p.slices, list[y]);
      const int first = max(sa.q0, sb.q0);
      if (first < a0 || first >= a1 || first >= min(sa.q1, sb.q1)) continue;
      if (max(sa.k0, sb.k0) >= min(sa.k1, sb.k1)) continue;
      if (pair_overlaps(sa, sb)) atomicOr(&p.hdr->status, FFA_META_ERR_OVERLAP);
    }
  }
}

// Block-wide exclusive scan of one int per thread (MT threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ int block_exclusive_scan(int x, int* lds_ws, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds_ws[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < MT / 64; ++i) {
    int v = lds_ws[i];
    if (i < w) base += v;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// One owner block of the q2k (DIR = 0) or k2q (DIR = 1) classification.
// FILL = false: write the Full / Partial counts of the owner (and, for q2k,
// its slice count and area).  FILL = true: write the ascending index lists.
struct TilesLds {
  int cnt[CH];
  int diff[CH + 1];
  int slist[MT];
  int ws[MT / 64 + 1];
  int minmax[2];
  long long area[MT / 64];
};

template <int DIR, bool FILL>
__device__ void tiles_block(void* meta, int own, TilesLds& sm) {
  int* const cnt = sm.cnt;
  int* const diff = sm.diff;
  int* const slist = sm.slist;
  int* const ws = sm.ws;
  int* const sh_minmax = sm.minmax;

  MetaPtrs p = meta_ptrs(meta);
  const MetaHeader* h = p.hdr;
  const int S = h->num_slices, Tq = h->seqlen_q, Tk = h->seqlen_k;
  // owner axis A and iterated axis B
  const int BA = DIR == 0 ? BM_F : BN_B;
  const int BB = DIR == 0 ? BN_F : BM_B;
  const int TA = DIR == 0 ? Tq : Tk;
  const int a0 = own * BA, a1 = min(a0 + BA, TA);
  const int cap = (a1 - a0) * BB;     // valid count of a Full tile
  const int tid = threadIdx.x;

  int32_t* full_off = DIR == 0 ? p.qf_off : p.kf_off;
  int32_t* mask_off = DIR == 0 ? p.qm_off : p.km_off;
  const int64_t capacity = h->capacity;
  int out_f = 0, out_p = 0;   // running positions (FILL)
  int64_t base_f = 0, base_p = 0;
  if (FILL) {
    base_f = h->list_off[DIR == 0 ? L_QF : L_KF] + full_off[own];
    base_p = h->list_off[DIR == 0 ? L_QM : L_KM] + mask_off[own];
  }

  // pass 1: iterated-block range touched by slices meeting this owner block,
  // and (q2k) the owner's slice list
  if (tid == 0) {
    sh_minmax[0] = 0x7fffffff;
    sh_minmax[1] = -1;
  }
  __syncthreads();
  int nslices_here = 0;
  int64_t qs_base = 0;
  if (FILL && DIR == 0) qs_base = h->list_off[L_QS] + p.qs_off[own];
  for (int sb = 0; sb < S; sb += MT) {
    const int si = sb + tid;
    int hit = 0;
    if (si < S) {
      const Slice s = load_slice(p.slices, si);
      if (slice_ok(s, Tq, Tk) && s.q1 > s.q0 && s.k1 > s.k0) {
        const int sa0 = DIR == 0 ? s.q0 : s.k0, sa1 = DIR == 0 ? s.q1 : s.k1;
        const int sb0 = DIR == 0 ? s.k0 : s.q0, sb1 = DIR == 0 ? s.k1 : s.q1;
        if (sa0 < a1 && sa1 > a0) {
          hit = 1;
          atomicMin(&sh_minmax[0], sb0 / BB);
          atomicMax(&sh_minmax[1], (sb1 - 1) / BB);
        }
      }
    }
    if (DIR == 0) {
      int tot;
      const int pos = block_exclusive_scan(hit, ws, &tot);
      if (FILL && hit) {
        const int64_t at = qs_base + nslices_here + pos;
        if (at < capacity) p.var[at] = si;
      }
      nslices_here += tot;
    }
  }
  __syncthreads();
  const int bmin = sh_minmax[0], bmax = sh_minmax[1];
  if (!FILL && DIR == 0 && tid == 0) p.qs_off[own + 1] = nslices_here;
  // the block's slice list is complete (the barrier above also makes its
  // global writes visible to the whole workgroup); it is only whole when the
  // lists fit the buffer, which the scan launch has decided
  if (FILL && DIR == 0 && (h->status & FFA_META_ERR_CAPACITY) == 0)
    validate_pairs(p, p.var + qs_base, nslices_here, a0, a1);

  int64_t area = 0;
  for (int cb0 = bmin; cb0 <= bmax; cb0 += CH) {
    const int cb1 = min(cb0 + CH, bmax + 1);   // blocks [cb0, cb1)
    const int nb = cb1 - cb0;
    // only the chunk's nb entries are used (intervals write below nb); the
    // rest of the arrays is never read
    for (int i = tid; i < nb; i += MT) {
      cnt[i] = 0;
      diff[i] = 0;
    }
    __syncthreads();
    const int lo_lim = cb0 * BB, hi_lim = cb1 * BB - 1;
    for (int sb = 0; sb < S; sb += MT) {
      // compact the slices of this group that meet the owner block
      const int si = sb + tid;
      int hit = 0;
      if (si < S) {
        const Slice s = load_slice(p.slices, si);
        if (slice_ok(s, Tq, Tk) && s.q1 > s.q0 && s.k1 > s.k0) {
          const int sa0 = DIR == 0 ? s.q0 : s.k0, sa1 = DIR == 0 ? s.q1 : s.k1;
          const int sb0 = DIR == 0 ? s.k0 : s.q0, sb1 = DIR == 0 ? s.k1 : s.q1;
          hit = (sa0 < a1 && sa1 > a0 && sb0 <= hi_lim && sb1 > lo_lim) ? 1 : 0;
        }
      }
      int tot;
      const int pos = block_exclusive_scan(hit, ws, &tot);
      if (hit) slist[pos] = si;
      __syncthreads();
      // every (slice, owner position) pair adds its interval
      for (int w = tid; w < tot * BA; w += MT) {
        const int pa = a0 + (w % BA);
        if (pa >= a1) continue;
        const Slice s = load_slice(p.slices, slist[w / BA]);
        int lo, hi;
        if (DIR == 0) row_interval(s, pa, lo, hi);
        else col_interval(s, pa, lo, hi);
        lo = max(lo, lo_lim);
        hi = min(hi, hi_lim);
        if (lo > hi) continue;
        const int bl = lo / BB - cb0, bh = hi / BB - cb0;
        if (bl == bh) {
          atomicAdd(&cnt[bl], hi - lo + 1);
        } else {
          atomicAdd(&cnt[bl], (bl + cb0 + 1) * BB - lo);
          atomicAdd(&cnt[bh], hi - (bh + cb0) * BB + 1);
          if (bh > bl + 1) {
            atomicAdd(&diff[bl + 1], BB);
            atomicAdd(&diff[bh], -BB);
          }
        }
      }
      __syncthreads();
    }
    // prefix sum of diff over the chunk: thread tid owns PER consecutive blocks
    int run = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) run += (tid * PER + e < nb) ? diff[tid * PER + e] : 0;
    int dummy;
    int carry = block_exclusive_scan(run, ws, &dummy);
    int nf = 0, np = 0;
    int vals[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int b = tid * PER + e;
      carry += (b < nb) ? diff[b] : 0;
      const int v = (b < nb) ? cnt[b] + carry : 0;
      vals[e] = v;
      area += v;
      nf += (v != 0 && v == cap);
      np += (v != 0 && v != cap);
    }
    int tf, tp;
    const int pf = block_exclusive_scan(nf, ws, &tf);
    const int pp = block_exclusive_scan(np, ws, &tp);
    if (FILL) {
      int of = out_f + pf, op = out_p + pp;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int v = vals[e];
        const int bidx = cb0 + tid * PER + e;
        if (v != 0 && v == cap) {
          const int64_t at = base_f + of++;
          if (at < capacity) p.var[at] = bidx;
        } else if (v != 0) {
          const int64_t at = base_p + op++;
          if (at < capacity) p.var[at] = bidx;
        }
      }
    }
    out_f += tf;
    out_p += tp;
    __syncthreads();
  }
  if (FILL) {
    // This owner's place in the longest-first schedule (owners with more work
    // first, ties by index; work = 4 per Full tile + 5 per Partial tile),
    // counted by all threads over all owners, and its block record.
    const int n = DIR == 0 ? h->nq_f : h->nk_b;
    auto cost = [&](int x) { return 4 * (full_off[x + 1] - full_off[x]) + 5 * (mask_off[x + 1] - mask_off[x]); };
    const int c = cost(own);
    int before = 0;
    if (n <= MAX_SORT)
      for (int x = tid; x < n; x += MT) {
        const int cx = cost(x);
        before += (cx > c) || (cx == c && x < own);
      }
    int rank;
    block_exclusive_scan(before, ws, &rank);
    if (n > MAX_SORT) rank = own;
    // (the scan's barriers also make this block's list entries visible here)
    if (tid == 0) {
      const int f0 = full_off[own], nF = full_off[own + 1] - f0;
      const int p0 = mask_off[own], nP = mask_off[own + 1] - p0;
      const int64_t lf = h->list_off[DIR == 0 ? L_QF : L_KF] + f0;
      const int64_t lp = h->list_off[DIR == 0 ? L_QM : L_KM] + p0;
      auto entry = [&](int64_t at) { return at < capacity ? p.var[at] : -1; };
      int32_t* r = (DIR == 0 ? p.rec_f : p.rec_b) + (int64_t)REC * rank;
      (DIR == 0 ? p.sched_f : p.sched_b)[rank] = own;
      r[R_OWNER] = own;
      r[R_F0] = f0;
      r[R_NF] = nF;
      r[R_P0] = p0;
      r[R_NP] = nP;
      if (DIR == 0) {
        r[R_S0] = p.qs_off[own];
        r[R_NS] = p.qs_off[own + 1] - p.qs_off[own];
        r[R_TF] = nF > 0 ? entry(lf) : -1;
        r[R_TP] = nP > 0 ? entry(lp) : -1;
      } else {
        r[RB_TF] = nF > 0 ? entry(lf + nF - 1) : -1;
        r[RB_TP] = nP > 0 ? entry(lp + nP - 1) : -1;
      }
    }
  }
  if (!FILL) {
    if (tid == 0) {
      full_off[own + 1] = out_f;
      mask_off[own + 1] = out_p;
    }
    if (DIR == 0) {
      // block-reduce the area (int64) and add once per owner
      long long* const sarea = sm.area;
      long long x = area;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
      if ((tid & 63) == 0) sarea[tid >> 6] = x;
      __syncthreads();
      if (tid == 0) {
        long long t = 0;
        for (int i = 0; i < MT / 64; ++i) t += sarea[i];
        if (t) atomicAdd(reinterpret_cast<unsigned long long*>(&p.hdr->area),
                         static_cast<unsigned long long>(t));
      }
    }
  }
}


// The five offset arrays (counts stored at [1..n]) turned into offsets in
// place, all five per chunk of blockDim.x entries: the chunk's values of every
// array are loaded before any is scanned, so a chunk waits for memory once,
// not five times.
__global__ void meta_scan_kernel(void* meta) {
  __shared__ int ws[5][16];
  MetaPtrs p = meta_ptrs(meta);
  MetaHeader* h = p.hdr;
  int32_t* const arr[5] = {p.qf_off, p.qm_off, p.kf_off, p.km_off, p.qs_off};
  const int len[5] = {h->nq_f, h->nq_f, h->nk_b, h->nk_b, h->nq_f};
  const int tid = threadIdx.x, NT = blockDim.x;
  const int lane = tid & 63, w = tid >> 6;
  const int nmax = max(h->nq_f, h->nk_b);
  if (tid == 0)
    for (int k = 0; k < 5; ++k) arr[k][0] = 0;
  int carry[5] = {0, 0, 0, 0, 0};
  for (int base = 1; base <= nmax; base += NT) {
    const int i = base + tid;
    int incl[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) incl[k] = (i <= len[k]) ? arr[k][i] : 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl[k], o, 64);
        if (lane >= o) incl[k] += y;
      }
      if (lane == 63) ws[k][w] = incl[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      int pre = 0, tot = 0;
      for (int q = 0; q < NT / 64; ++q) {
        if (q < w) pre += ws[k][q];
        tot += ws[k][q];
      }
      if (i <= len[k]) arr[k][i] = carry[k] + pre + incl[k];
      carry[k] += tot;
    }
    __syncthreads();
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t n0 = p.qf_off[h->nq_f], n1 = p.qm_off[h->nq_f];
    const int64_t n2 = p.kf_off[h->nk_b], n3 = p.km_off[h->nk_b];
    const int64_t n4 = p.qs_off[h->nq_f];
    h->nnz[0] = n0;
    h->nnz[1] = n1;
    h->nnz[2] = n2;
    h->nnz[3] = n3;
    h->nnz[4] = n4;
    h->list_off[0] = 0;
    h->list_off[1] = n0;
    h->list_off[2] = n0 + n1;
    h->list_off[3] = n0 + n1 + n2;
    h->list_off[4] = n0 + n1 + n2 + n3;
    if (n0 + n1 + n2 + n3 + n4 > h->capacity) atomicOr(&h->status, FFA_META_ERR_CAPACITY);
  }
}

// Counting launch: blocks [0, nq_f) count q2k owners, the next nk_b count k2q
// owners, the rest check the slices' bounds and types (MT slices each).
__global__ __launch_bounds__(MT) void meta_count_kernel(void* meta, int nq, int nk) {
  __shared__ TilesLds sm;
  const int b = blockIdx.x;
  if (b < nq) tiles_block<0, false>(meta, b, sm);
  else if (b < nq + nk) tiles_block<1, false>(meta, b - nq, sm);
  else check_slices(meta, b - nq - nk);
}

// Filling launch: blocks [0, nq_f) fill q2k lists, test the disjointness of
// the slice pairs whose common rows begin in their block and place their
// block in the forward schedule; the next nk_b do the same for the k2q lists
// and the backward schedule.
__global__ __launch_bounds__(MT) void meta_fill_kernel(void* meta, int nq, int nk) {
  __shared__ TilesLds sm;
  const int b = blockIdx.x;
  if (b < nq) tiles_block<0, true>(meta, b, sm);
  else tiles_block<1, true>(meta, b - nq, sm);
}

}  // namespace

hipError_t launch_build_meta(const int32_t* d_slices, int32_t S, int32_t Tq, int32_t Tk,
                             int32_t head_dim, void* d_meta, int64_t capacity,
                             const MetaLayout& L, hipStream_t stream) {
  InitArgs ia;
  ia.S = S;
  ia.Tq = Tq;
  ia.Tk = Tk;
  ia.head_dim = head_dim;
  ia.nq_f = L.nq_f;
  ia.nk_f = L.nk_f;
  ia.nq_b = L.nq_b;
  ia.nk_b = L.nk_b;
  ia.capacity = capacity;
  for (int i = 0; i < 11; ++i) ia.byte_off[i] = L.byte_off[i];
  const int n5 = 5 * S;
  const int gi = n5 > 0 ? min(1024, (n5 + 255) / 256) : 1;
  // four launches: init | count + slice checks | scan | fill + pair checks +
  // schedules and block recordss
  meta_init_kernel<<<gi, 256, 0, stream>>>(d_slices, d_meta, ia);
  const int nv = (S + MT - 1) / MT;
  if (L.nq_f + L.nk_b + nv > 0)
    meta_count_kernel<<<L.nq_f + L.nk_b + nv, MT, 0, stream>>>(d_meta, L.nq_f, L.nk_b);
  meta_scan_kernel<<<1, 1024, 0, stream>>>(d_meta);
  if (L.nq_f + L.nk_b > 0)
    meta_fill_kernel<<<L.nq_f + L.nk_b, MT, 0, stream>>>(d_meta, L.nq_f, L.nk_b);
  return hipGetLastError();
}

}  // namespace ffa
