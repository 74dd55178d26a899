// prefill_seg.hip -- segment-parallel carry of the chunked prefill (bf16
// operands, chunk 32 or 64) on gfx950.
//
// Per chunk the state obeys the affine recurrence (notation of prefill.hip)
//
//   S' = e^{gamma_last} S + K^T diag(c) Tt (V - diag(a) K S)  =  M S + B,
//
// with M = e^{gamma_last} I - K^T diag(c) Tt diag(a) K independent of the
// state.  The oxydllm 0.0.0-alpha.12.2 notes ("Performance", Gated DeltaNet
// fast paths) make the cross-chunk loop cheap by precomputing everything
// state-independent in batch; the loop itself stays sequential.  With one
// sequence that loop is 64 chunks deep per head, far too little parallel
// work for 256 compute units, so every sequence is cut into segments of
// seg_len chunks and the carry runs in three launches:
//
//   pass 1  (one workgroup per segment and v-head, all but the last segment
//           of a sequence) carries Z = [S | Phi] through the segment: S from
//           zero (the true initial state for the first segment) and Phi from
//           the identity, i.e. the segment's B and its transition
//           Phi = M_last ... M_first.  Both go to the workspace.
//   combine (one workgroup per sequence, v-head and 16 state columns) chains
//           the segment starts: S_start[p+1] = Phi_p S_start[p] + B_p.
//   pass 2  (one workgroup per segment and v-head) re-runs each segment from
//           its true start state and writes the outputs
//           O = diag(b) Q S + P U, and the final state.
//
// A workgroup holds a whole head (all d_v columns), so every chunk's K, Q,
// V, Tt and P are staged into LDS once per pass, not once per column tile.
// Four waves split the state columns; each keeps its slice of S (and Phi)
// in fp32 MFMA accumulators for the whole segment and feeds it back as bf16
// operands (gdn_device.h, MFMA fragment helpers).  Loads of chunk i+2 are in
// flight while chunk i is computed; LDS is double-buffered with one barrier
// per chunk.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ int nseg_of(int nchunks, int L) { return nchunks > 0 ? (nchunks + L - 1) / L : 1; }

struct Seg {
  int seq, p, nseg;   // sequence, segment index in it, its segment count
  int s0, s1;         // token range of the sequence
  int cbase, sbase;   // first global chunk and first global segment of the sequence
};

// Global segment n (grids are sized by a bound: seq == -1 past the last one).
__device__ __forceinline__ Seg seg_of(const ScanArgs& a, int C, int n) {
  Seg g;
  if (a.seqlen > 0) {
    const int cps = (a.seqlen + C - 1) / C;
    const int ns = nseg_of(cps, a.seg_len);
    const int seq = n / ns;
    g.seq = seq < a.num_seqs ? seq : -1;
    g.p = n - seq * ns;
    g.nseg = ns;
    g.s0 = seq * a.seqlen;
    g.s1 = g.s0 + a.seqlen;
    g.cbase = seq * cps;
    g.sbase = seq * ns;
    return g;
  }
  const int total = a.seg_offsets[a.num_seqs];
  int lo = 0, hi = a.num_seqs - 1;  // last sequence with seg_offsets[seq] <= n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.seg_offsets[mid] <= n) lo = mid; else hi = mid - 1;
  }
  g.seq = n < total ? lo : -1;
  g.sbase = a.seg_offsets[lo];
  g.p = n - g.sbase;
  g.nseg = a.seg_offsets[lo + 1] - g.sbase;
  g.s0 = a.cu_seqlens[lo];
  g.s1 = a.cu_seqlens[lo + 1];
  g.cbase = a.chunk_offsets[lo];
  return g;
}

// Block -> (global segment, v-head).  The G v-heads reading one q/k head in
// one segment get the same blockIdx % 8, i.e. the same XCD, and share its L2
// for K and Q.  With variable lengths the segments are taken in the order
// the chunk table chose (longest first): the passes hold one workgroup per
// compute unit, so a long chain dispatched late would set the end time.
__device__ __forceinline__ void block_unit(const ScanArgs& a, int& n, int& hk, int& h) {
  const int G = a.hv / a.hk;
  const int xcd = blockIdx.x & 7, m8 = blockIdx.x >> 3;
  const int grp = (m8 / G) * 8 + xcd;
  const int vh = m8 % G;
  n = grp / a.hk;
  hk = grp % a.hk;
  h = a.tiled ? (hk + vh * a.hk) : (hk * G + vh);
  if (a.seg_perm && n < a.seg_offsets[a.num_seqs]) n = a.seg_perm[n];
}

__device__ __forceinline__ uint16_t bf16_rne(float x) { return (uint16_t)(cvt_bf16x2(x, 0.f) & 0xffffu); }

// Workspace images of segment data, laid out as the registers that use them
// so that every access is one 16-byte word per lane:
//  - a d_k x d_v fp32 state in accumulator form: tile (u, jt) (rows 16u..,
//    columns 16jt..) is 64 lanes x f32x4, lane (c, g) holding rows 16u+4g+e
//    of column 16jt+c;
//  - a d_k x d_k bf16 transition as matrix-core A operands: fragment (u, m)
//    (rows 16u.., k = 32m..) is 64 lanes x 8 bf16, lane (c, g) holding row
//    16u+c at k = 32m + {4g+e, 16+4g+e}.
template <int DV>
__device__ __forceinline__ long state_frag(int u, int jt, int lane) {
  return ((long)(u * (DV / 16) + jt) * 64 + lane) * 4;
}
template <int DK>
__device__ __forceinline__ long phi_frag(int u, int m, int lane) {
  return ((long)(u * (DK / 32) + m) * 64 + lane) * 8;
}

// LDS image of one chunk.  K and Q (and Tt, P) rows are stored with the
// column permutation of perm_lo, V rows as they are.
template <int C, int DK, int DV, bool OUT>
struct alignas(16) SegSmem {
  static constexpr int KLD = DK + 16;  // row pads keep 16-byte fragment reads conflict-free
  static constexpr int VLD = DV + 16;
  static constexpr int CLD = C + 8;
  uint16_t k[2][C][KLD];
  uint16_t v[2][C][VLD];
  uint16_t tt[2][C][CLD];
  float sc[2][OUT ? kScalRows : 4][C];  // per-row scalars (rows as in the workspace; pass 2 puts scale rq in row 6)
  uint16_t q[OUT ? 2 : 1][OUT ? C : 1][KLD];
  uint16_t p[OUT ? 2 : 1][OUT ? C : 1][CLD];
};

// Global -> register -> LDS staging of one chunk by the NTH threads of a
// workgroup.  Rows of K, Q, V past the end of the sequence read as zero.
template <int C, int DK, int DV, bool OUT, int NTH>
struct Stager {
  typedef SegSmem<C, DK, DV, OUT> SM;
  // 16-byte vectors; Tt comes as its NLOW lower 16x16 blocks, packed (block
  // n = t(t+1)/2 + j, row-major, 32 vectors each)
  static constexpr int NRT = C / 16, NLOW = NRT * (NRT + 1) / 2;
  static constexpr int KV = C * DK / 8, VV = C * DV / 8, TV = NLOW * 32;
  static constexpr int NK = (KV + NTH - 1) / NTH, NV = (VV + NTH - 1) / NTH, NT = (TV + NTH - 1) / NTH;
  u32x4 rk[NK], rq[OUT ? NK : 1], rv[NV], rt[NT], rs;
  int tt_off[NT];  // LDS element offset (row, permuted column) of each Tt vector, the same for every chunk
  // this thread's K, Q and V vectors: row within the chunk (C, never loaded,
  // past the arrays) and element offset from the chunk's first row, the same
  // for every chunk
  int krow[NK], vrow[NV];
  long koff[NK], qoff[OUT ? NK : 1], voff[NV];
  const uint16_t *kp, *qp, *vp, *mp;
  const float* sp;
  long sk, sq, sv, mstep, sstep;
  int ntok, tid, l2norm;
  float scale;
  // the fused norm's gate rows z, staged like V (in V's buffer once the
  // carry is done with V)
  u32x4 rz[OUT ? NV : 1];
  long zoff[OUT ? NV : 1];
  const uint16_t* zp;

  __device__ __forceinline__ void setup_z(const uint16_t* z, long stride_z) {
    zp = z;
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int idx = tid + NTH * j, r = idx / (DV / 8), cv = idx % (DV / 8);
      zoff[j] = (long)r * stride_z + 8 * cv;
    }
  }
  __device__ __forceinline__ void zload(int ch, long stride_z) {
    const int cs = ch * C;
    const int clen = min(C, ntok - cs);
    const uint16_t* zc = zp + (long)cs * stride_z;
#pragma unroll
    for (int j = 0; j < NV; j++)
      rz[j] = vrow[j] < clen ? *reinterpret_cast<const u32x4*>(zc + zoff[j]) : u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void zstore(SM& sm, int b) const {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int idx = tid + NTH * j, r = idx / (DV / 8), cv = idx % (DV / 8);
      if (idx < VV) *reinterpret_cast<u32x4*>(&sm.v[b][r][8 * cv]) = rz[j];
    }
  }

  __device__ __forceinline__ void setup_offsets() {
#pragma unroll
    for (int j = 0; j < NK; j++) {
      const int idx = tid + NTH * j, r = idx / (DK / 8), cv = idx % (DK / 8);
      krow[j] = idx < KV ? r : C;
      koff[j] = (long)r * sk + 8 * cv;
      if constexpr (OUT) qoff[j] = (long)r * sq + 8 * cv;
    }
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int idx = tid + NTH * j, r = idx / (DV / 8), cv = idx % (DV / 8);
      vrow[j] = idx < VV ? r : C;
      voff[j] = (long)r * sv + 8 * cv;
    }
  }

  __device__ __forceinline__ void load(int ch) {  // ch: chunk index within the sequence
    const int cs = ch * C;
    const int clen = min(C, ntok - cs);
    const uint16_t* kc = kp + (long)cs * sk;
    const uint16_t* qc = qp + (long)cs * sq;
    const uint16_t* vc = vp + (long)cs * sv;
#pragma unroll
    for (int j = 0; j < NK; j++) {
      const bool ok = krow[j] < clen;
      rk[j] = ok ? *reinterpret_cast<const u32x4*>(kc + koff[j]) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (OUT) rq[j] = ok ? *reinterpret_cast<const u32x4*>(qc + qoff[j]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NV; j++)
      rv[j] = vrow[j] < clen ? *reinterpret_cast<const u32x4*>(vc + voff[j]) : u32x4{0u, 0u, 0u, 0u};
    const uint16_t* mc = mp + ch * mstep;
#pragma unroll
    for (int j = 0; j < NT; j++) {
      const int idx = tid + NTH * j;
      if (idx < TV) rt[j] = *reinterpret_cast<const u32x4*>(mc + 8 * idx);
    }
    // scalar rows 0..3 (and 4..7 with outputs)
    if (tid < (OUT ? 2 : 1) * C) rs = *reinterpret_cast<const u32x4*>(sp + ch * sstep + 4 * tid);
  }

  __device__ __forceinline__ void store(SM& sm, int b) const {
#pragma unroll
    for (int j = 0; j < NK; j++) {
      const int idx = tid + NTH * j, r = idx / (DK / 8), lo = perm_lo(idx % (DK / 8));
      if (idx < KV) {
        *reinterpret_cast<u32x2*>(&sm.k[b][r][lo]) = u32x2{rk[j][0], rk[j][1]};
        *reinterpret_cast<u32x2*>(&sm.k[b][r][lo + 8]) = u32x2{rk[j][2], rk[j][3]};
        if constexpr (OUT) {
          *reinterpret_cast<u32x2*>(&sm.q[b][r][lo]) = u32x2{rq[j][0], rq[j][1]};
          *reinterpret_cast<u32x2*>(&sm.q[b][r][lo + 8]) = u32x2{rq[j][2], rq[j][3]};
        }
      }
      if constexpr (OUT) {
        // scale / |q_r| (row 6): the DK/8 words of a row sit in consecutive lanes
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) ss = dot2_bf16(rq[j][e], rq[j][e], ss);
        ss = group_sum<DK / 8>(ss);
        if (idx < KV && idx % (DK / 8) == 0)
          sm.sc[b][6][r] = scale * (l2norm ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.0f);
      }
    }
#pragma unroll
    for (int j = 0; j < NV; j++) {
      const int idx = tid + NTH * j, r = idx / (DV / 8), cv = idx % (DV / 8);
      if (idx < VV) *reinterpret_cast<u32x4*>(&sm.v[b][r][8 * cv]) = rv[j];
    }
#pragma unroll
    for (int j = 0; j < NT; j++) {
      if (TV % NTH == 0 || tid + NTH * j < TV) {
        uint16_t* d = &sm.tt[b][0][0] + tt_off[j];
        *reinterpret_cast<u32x2*>(d) = u32x2{rt[j][0], rt[j][1]};
        *reinterpret_cast<u32x2*>(d + 8) = u32x2{rt[j][2], rt[j][3]};
      }
    }
    // row 6 is this stager's own (scale rq, above)
    if (tid < (OUT ? 2 : 1) * C && (4 * tid) / C != 6) *reinterpret_cast<u32x4*>(&sm.sc[b][0][0] + 4 * tid) = rs;
  }

  // Where each of this thread's packed Tt vectors goes in a chunk buffer
  // (vector idx: block n = idx / 32, its row (idx % 32) / 2, half idx % 2),
  // and zeros in the upper blocks (t, t + 1), t even, of both buffers: the
  // carry's 32-wide k steps read them, the workspace does not hold them and
  // no chunk's store touches them.  Once, before the first store.
  __device__ __forceinline__ void setup_tt(SM& sm) {
#pragma unroll
    for (int j = 0; j < NT; j++) {
      const int idx = tid + NTH * j;
      const int n = idx < TV ? idx >> 5 : 0, rr = (idx & 31) >> 1, w = idx & 1;
      int t = 0;
      while ((t + 1) * (t + 2) / 2 <= n) t++;
      tt_off[j] = (16 * t + rr) * SM::CLD + perm_lo(2 * (n - t * (t + 1) / 2) + w);
    }
    constexpr int NZW = 2 * (NRT / 2) * 32;  // (buffer, block, row, half)
    for (int idx = tid; idx < NZW; idx += NTH) {
      const int w = idx & 1, rr = (idx >> 1) & 15, z = (idx >> 5) % (NRT / 2), b = idx / (NRT / 2 * 32);
      const int t = 2 * z, lo = perm_lo(2 * (t + 1) + w);
      *reinterpret_cast<u32x2*>(&sm.tt[b][16 * t + rr][lo]) = u32x2{0u, 0u};
      *reinterpret_cast<u32x2*>(&sm.tt[b][16 * t + rr][lo + 8]) = u32x2{0u, 0u};
    }
  }
};

// One chunk of the carry for the NCT 16-column tiles of Z owned by this
// wave (tile j is state column tile col[j]; vcol[j] < 0 marks a transition
// tile, whose values term is zero).  Z <- e^{gl} Z + K^T diag(c) Tt (V -
// diag(a) K Z).  With OUT, also O^T = (Z^T Q^T) diag(b) + U^T P^T, returned in
// ob as bf16: lane (c16, g) holds columns 4g..4g+3 of tile j for token 16t+c16.
// mid() runs after the state update, before P is read.
template <int C, int DK, int DV, int NCT, bool OUT, class Mid>
__device__ __forceinline__ void carry_chunk(SegSmem<C, DK, DV, OUT>& sm, int b, f32x4 (&Z)[DK / 16][NCT],
                                            const int (&vcol)[NCT], int lane, u32x2 (&ob)[NCT][C / 16], Mid mid) {
  typedef SegSmem<C, DK, DV, OUT> SM;
  constexpr int NRT = C / 16, PS = C / 32, KS = DK / 32, NDT = DK / 16;
  const int c16 = lane & 15, g = lane >> 4, r4 = 4 * g;

  // Z as bf16 operand fragments, k = d_k rows 32m + {4g+e, 16+4g+e}
  bf16x8 zb[KS][NCT];
#pragma unroll
  for (int m = 0; m < KS; m++)
#pragma unroll
    for (int j = 0; j < NCT; j++) zb[m][j] = frag_acc(Z[2 * m][j], Z[2 * m + 1][j]);

  // X = K Z
  f32x4 X[NRT][NCT];
#pragma unroll
  for (int t = 0; t < NRT; t++)
#pragma unroll
    for (int j = 0; j < NCT; j++) X[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < KS; m++)
#pragma unroll
    for (int t = 0; t < NRT; t++) {
      const bf16x8 ak = ld_frag(&sm.k[b][16 * t + c16][32 * m + 8 * g]);
#pragma unroll
      for (int j = 0; j < NCT; j++) X[t][j] = mfma16(ak, zb[m][j], X[t][j]);
    }

  // R = V - diag(a) X  (lane: tokens 16t + 4g + e of column c16 of the tile)
#pragma unroll
  for (int t = 0; t < NRT; t++) {
    const f32x4 av = ld4(&sm.sc[b][0][16 * t + r4]);
#pragma unroll
    for (int j = 0; j < NCT; j++) {
      f32x4 vv = {0.f, 0.f, 0.f, 0.f};
      if (vcol[j] >= 0) vv = bf4_to_f32(ld_tr(&sm.v[b][16 * t + r4 + (c16 >> 2)][vcol[j] + 4 * (c16 & 3)]));
      X[t][j] = vv - av * X[t][j];
    }
  }

  // U = Tt R (Tt lower triangular by 16-row blocks: row tile t needs k steps pp <= t/2)
  f32x4 U[NRT][NCT];
#pragma unroll
  for (int t = 0; t < NRT; t++)
#pragma unroll
    for (int j = 0; j < NCT; j++) U[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int pp = 0; pp < PS; pp++) {
    bf16x8 rb[NCT];
#pragma unroll
    for (int j = 0; j < NCT; j++) rb[j] = frag_acc(X[2 * pp][j], X[2 * pp + 1][j]);
#pragma unroll
    for (int t = 2 * pp; t < NRT; t++) {
      const bf16x8 at = ld_frag(&sm.tt[b][16 * t + c16][32 * pp + 8 * g]);
#pragma unroll
      for (int j = 0; j < NCT; j++) U[t][j] = mfma16(at, rb[j], U[t][j]);
    }
  }

  // With OUT: O^T = (Z^T Q^T) diag(b) + U^T P^T, b = (scale rq) e^{gamma}; lane
  // (c16, g) holds 4 consecutive columns 4g..4g+3 of token 16t + c16.  Only
  // the last term needs P, so it comes after mid() and after the state
  // update; the unscaled U is kept as operand fragments for it.
  f32x4 Y[OUT ? NCT : 1][OUT ? NRT : 1];
  bf16x8 uo[OUT ? PS : 1][NCT];
  if constexpr (OUT) {
#pragma unroll
    for (int j = 0; j < NCT; j++)
#pragma unroll
      for (int t = 0; t < NRT; t++) Y[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KS; m++)
#pragma unroll
      for (int t = 0; t < NRT; t++) {
        const bf16x8 bq = ld_frag(&sm.q[b][16 * t + c16][32 * m + 8 * g]);
#pragma unroll
        for (int j = 0; j < NCT; j++) Y[j][t] = mfma16(zb[m][j], bq, Y[j][t]);
      }
#pragma unroll
    for (int t = 0; t < NRT; t++) {
      const float bt = sm.sc[b][6][16 * t + c16] * sm.sc[b][7][16 * t + c16];
#pragma unroll
      for (int j = 0; j < NCT; j++) Y[j][t] = bt * Y[j][t];
    }
#pragma unroll
    for (int pp = 0; pp < PS; pp++)
#pragma unroll
      for (int j = 0; j < NCT; j++) uo[pp][j] = frag_acc(U[2 * pp][j], U[2 * pp + 1][j]);
  }

  // Z <- e^{gamma_last} Z + K^T (diag(c) U)
#pragma unroll
  for (int t = 0; t < NRT; t++) {
    const f32x4 cv = ld4(&sm.sc[b][2][16 * t + r4]);
#pragma unroll
    for (int j = 0; j < NCT; j++) U[t][j] = cv * U[t][j];
  }
  const float gl = sm.sc[b][3][0];
#pragma unroll
  for (int u = 0; u < NDT; u++)
#pragma unroll
    for (int j = 0; j < NCT; j++) Z[u][j] = gl * Z[u][j];
#pragma unroll
  for (int pp = 0; pp < PS; pp++) {
    bf16x8 ub[NCT];
#pragma unroll
    for (int j = 0; j < NCT; j++) ub[j] = frag_acc(U[2 * pp][j], U[2 * pp + 1][j]);
#pragma unroll
    for (int u = 0; u < NDT; u++) {
      // K^T fragment: lane (c16, g) gets K[32pp + {4g+e, 16+4g+e}][16u + c16]
      const uint16_t* p0 = &sm.k[b][32 * pp + r4 + (c16 >> 2)][32 * (u >> 1) + 8 * (c16 & 3) + 4 * (u & 1)];
      const bf16x8 akt = frag2(ld_tr(p0), ld_tr(p0 + 16 * SM::KLD));
#pragma unroll
      for (int j = 0; j < NCT; j++) Z[u][j] = mfma16(akt, ub[j], Z[u][j]);
    }
  }

  mid();  // pass 2: P of this chunk is ready in LDS after this
  if constexpr (OUT) {
#pragma unroll
    for (int pp = 0; pp < PS; pp++) {
#pragma unroll
      for (int t = 2 * pp; t < NRT; t++) {
        const bf16x8 bp = ld_frag(&sm.p[b][16 * t + c16][32 * pp + 8 * g]);
#pragma unroll
        for (int j = 0; j < NCT; j++) Y[j][t] = mfma16(uo[pp][j], bp, Y[j][t]);
      }
    }
#pragma unroll
    for (int j = 0; j < NCT; j++)
#pragma unroll
      for (int t = 0; t < NRT; t++) ob[j][t] = pack4_bf16(Y[j][t]);
  }
}

// P of the chunk in LDS buffer b, formed by the NSW staging waves (sw = this
// wave among them) from the staged K and raw Q and the row scalars:
//   P[r][s] = (scale rq_r) rk_s e^{gamma_r - gamma_s} q_r . k_s   (s <= r), else 0,
// in the carry's operand layout: row r, column s at the permuted position.
// Tiles (t, j) with j <= t are products; the upper tiles (t even, j = t + 1)
// that a 32-wide k step also reads are written as zero.  Each tile is
// D = K_j Q_t^T on the matrix cores, so lane (c16, g) holds P[16t + c16][16j + 4g + e]:
// 4 consecutive columns, one 8-byte store.
template <int C, int DK, int DV, int NSW>
__device__ __forceinline__ void compute_p(SegSmem<C, DK, DV, true>& sm, int b, int sw, int lane) {
  constexpr int NRT = C / 16, KS = DK / 32;
  constexpr int NLOW = NRT * (NRT + 1) / 2, NZ = NRT / 2;
  const int c16 = lane & 15, g = lane >> 4, r4 = 4 * g;
  for (int n = sw; n < NLOW + NZ; n += NSW) {
    int t, j;
    bool zero = n >= NLOW;
    if (!zero) {
      t = 0;
      while ((t + 1) * (t + 2) / 2 <= n) t++;
      j = n - t * (t + 1) / 2;
    } else {
      t = 2 * (n - NLOW);
      j = t + 1;
    }
    const int r = 16 * t + c16, s0 = 16 * j + r4;
    u32x2 w = {0u, 0u};
    if (!zero) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KS; m++)
        acc = mfma16(ld_frag(&sm.k[b][16 * j + c16][32 * m + 8 * g]), ld_frag(&sm.q[b][r][32 * m + 8 * g]), acc);
      const float fr = sm.sc[b][6][r], gr = sm.sc[b][4][r];
      const f32x4 rks = ld4(&sm.sc[b][5][s0]), gs = ld4(&sm.sc[b][4][s0]);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = s0 + e <= r ? fr * rks[e] * __expf(gr - gs[e]) * acc[e] : 0.f;
      w = pack4_bf16(v);
    }
    // logical columns s0..s0+3 sit together at 32(j/2) + 8g + 4(j%2)
    *reinterpret_cast<u32x2*>(&sm.p[b][r][32 * (j >> 1) + 8 * g + 4 * (j & 1)]) = w;
  }
}

// Set up a stager for (segment g, heads hk / h).
template <int C, int DK, int DV, bool OUT, int NTH>
__device__ __forceinline__ void init_stager(Stager<C, DK, DV, OUT, NTH>& st, const ScanArgs& a, const Seg& sg, int hk,
                                            int h, int tid) {
  st.tid = tid;
  st.ntok = sg.s1 - sg.s0;
  st.sk = a.stride_k;
  st.sq = a.stride_q;
  st.sv = a.stride_v;
  st.kp = reinterpret_cast<const uint16_t*>(a.k) + (long)sg.s0 * a.stride_k + (long)hk * DK;
  st.qp = reinterpret_cast<const uint16_t*>(a.q) + (long)sg.s0 * a.stride_q + (long)hk * DK;
  st.vp = reinterpret_cast<const uint16_t*>(a.v) + (long)sg.s0 * a.stride_v + (long)h * DV;
  st.mp = reinterpret_cast<const uint16_t*>(a.tinv) + ((long)sg.cbase * a.hv + h) * (2 * C * C);
  st.sp = a.scal + ((long)sg.cbase * a.hv + h) * (kScalRows * C);
  st.mstep = (long)a.hv * (2 * C * C);
  st.sstep = (long)a.hv * (kScalRows * C);
  st.l2norm = a.l2norm;
  st.scale = a.scale;
  st.setup_offsets();
}

// ------------------------------------------------------------------ pass 1
template <int C, int DK, int DV, int NW>
__global__ void __launch_bounds__(64 * NW) k_seg_pass1(ScanArgs a) {
  typedef SegSmem<C, DK, DV, false> SM;
  constexpr int NDT = DK / 16;
  constexpr int NCT = (DV + DK) / (16 * NW);  // [S | Phi] column tiles per wave
  constexpr int SVT = DV / 16;                // tiles below SVT are state columns
  static_assert(NCT * 16 * NW == DV + DK, "columns must split over the waves");
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int c16 = lane & 15, r4 = 4 * (lane >> 4);
  int n, hk, h;
  block_unit(a, n, hk, h);
  const Seg sg = seg_of(a, C, n);
  if (sg.seq < 0 || sg.p >= sg.nseg - 1) return;  // the last segment needs no carry pass
  const int ch0 = sg.p * a.seg_len;
  const int nch = a.seg_len;  // every segment but the last is full

  int vcol[NCT];
  f32x4 Z[NDT][NCT];
  const float* sin = (sg.p == 0 && a.state_in) ? a.state_in + ((long)sg.seq * a.hv + h) * DK * DV : nullptr;
  float* sst = a.seg_state + ((long)(sg.sbase + sg.p) * a.hv + h) * DK * DV;
  // Z = [S | Phi]: S from state_in (first segment) or zero, Phi = I.  The
  // state_in branch encloses its whole loop so that its loads all issue
  // before the first wait.
#pragma unroll
  for (int j = 0; j < NCT; j++) {
    const int gt = wave * NCT + j;
    vcol[j] = gt < SVT ? 16 * gt : -1;
    const int col = gt < SVT ? 16 * gt + c16 : 16 * (gt - SVT) + c16;
#pragma unroll
    for (int u = 0; u < NDT; u++)
#pragma unroll
      for (int e = 0; e < 4; e++) Z[u][j][e] = (gt >= SVT && 16 * u + r4 + e == col) ? 1.f : 0.f;
  }
  if (sin) {
#pragma unroll
    for (int j = 0; j < NCT; j++) {
      const int gt = wave * NCT + j;
      if (gt < SVT) {
#pragma unroll
        for (int u = 0; u < NDT; u++)
#pragma unroll
          for (int e = 0; e < 4; e++) Z[u][j][e] = sin[(long)(16 * u + r4 + e) * DV + 16 * gt + c16];
      }
    }
  }
  // the first segment records its start state for pass 2 (the caller's
  // state_in may be overwritten by state_out meanwhile)
  if (sg.p == 0) {
#pragma unroll
    for (int j = 0; j < NCT; j++) {
      const int gt = wave * NCT + j;
      if (gt < SVT) {
#pragma unroll
        for (int u = 0; u < NDT; u++) *reinterpret_cast<f32x4*>(sst + state_frag<DV>(u, gt, lane)) = Z[u][j];
      }
    }
  }

  Stager<C, DK, DV, false, 64 * NW> st;
  init_stager(st, a, sg, hk, h, tid);
  st.load(ch0);
  st.setup_tt(sm);
  st.store(sm, 0);
  if (nch > 1) st.load(ch0 + 1);
  u32x2 ob[NCT][C / 16];
  for (int i = 0; i < nch; i++) {
    lds_barrier();
    const int b = i & 1;
    if (i + 1 < nch) st.store(sm, b ^ 1);
    if (i + 2 < nch) st.load(ch0 + i + 2);
    carry_chunk<C, DK, DV, NCT, false>(sm, b, Z, vcol, lane, ob, [] {});
  }

  // B_p (or the true end state of the first segment) is the next segment's
  // start before the combine
  float* snext = sst + (long)a.hv * DK * DV;
#pragma unroll
  for (int j = 0; j < NCT; j++) {
    const int gt = wave * NCT + j;
    if (gt < SVT) {
#pragma unroll
      for (int u = 0; u < NDT; u++) *reinterpret_cast<f32x4*>(snext + state_frag<DV>(u, gt, lane)) = Z[u][j];
    }
  }
  if (sg.p == 0) return;
  // Phi_p in bf16 as A-operand fragments: transposed through LDS (the chunk
  // buffers are free once every wave is past the last chunk)
  constexpr int PLD = DK + 8;
  uint16_t* img = reinterpret_cast<uint16_t*>(&sm);
  static_assert(sizeof(SM) >= DK * PLD * 2, "transition image must fit the chunk buffers");
  lds_barrier();
#pragma unroll
  for (int j = 0; j < NCT; j++) {
    const int gt = wave * NCT + j;
    if (gt >= SVT) {
#pragma unroll
      for (int u = 0; u < NDT; u++)
#pragma unroll
        for (int e = 0; e < 4; e++) img[(16 * u + r4 + e) * PLD + 16 * (gt - SVT) + c16] = bf16_rne(Z[u][j][e]);
    }
  }
  lds_barrier();
  uint16_t* phi = a.seg_phi + ((long)(sg.sbase + sg.p) * a.hv + h) * DK * DK;
  for (int f = wave; f < NDT * (DK / 32); f += NW) {
    const int u = f / (DK / 32), m = f % (DK / 32);
    const uint16_t* row = img + (16 * u + c16) * PLD + 32 * m + r4;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(row), hi = *reinterpret_cast<const u32x2*>(row + 16);
    *reinterpret_cast<u32x4*>(phi + phi_frag<DK>(u, m, lane)) = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
}

// ----------------------------------------------------------------- combine
// S_start[p+1] = Phi_p S_start[p] + B_p for p = 1 .. nseg-2, in place over
// B_p.  The chain is separable by state columns: one workgroup per
// (sequence, v-head, CW 16-column tiles), CW RS + LW waves:
//  - waves 0..CW RS-1 hold one 16-column tile of S (all rows) in registers,
//    so S feeds the matrix cores straight from them; RS waves share a tile
//    by rows of the product, each computing and storing its NDT / RS row
//    tiles and passing them to the others through LDS (parity-double-
//    buffered, ordered by the step's barrier); they only store;
//  - waves CW.. only load: Phi_p and the B_p columns, NS steps ahead in NS
//    register sets, into an NS-slot LDS ring.
// Keeping loads and stores in different waves means no wait for a load ever
// has to wait for a store to be acknowledged.  The column groups of one
// v-head get the same blockIdx % 8, i.e. the same XCD, and share its L2 for
// the transitions.
template <int DK, int DV, int CW, int RS, int LW, int NS>
__global__ void __launch_bounds__(64 * (CW * RS + LW)) k_seg_combine(ScanArgs a) {
  constexpr int NDT = DK / 16, KS = DK / 32;
  constexpr int UPR = NDT / RS;                             // row tiles per compute wave
  static_assert(UPR * RS == NDT, "row tiles must split over the row shares");
  constexpr int NG = DV / (16 * CW);                        // column groups per v-head
  constexpr int LT = 64 * LW;                               // loader threads
  constexpr int PV = DK * DK / 8 / LT;                      // 16-byte words of Phi per loader thread
  constexpr int BV = NDT * CW * 64 / LT;                    // f32x4 words of B per loader thread
  static_assert(PV * LT * 8 == DK * DK && BV * LT == NDT * CW * 64, "shape");
  __shared__ u32x4 phl[NS][DK * DK / 8];
  __shared__ f32x4 bl[NS][NDT * CW * 64];                   // [u][tile][lane]
  constexpr int SXN = RS > 1 ? 2 * CW * NDT * 64 : 1;
  __shared__ f32x4 sx[SXN];                                 // [parity][tile][u][lane]: rows passed between shares
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int xcd = blockIdx.x & 7, m8 = blockIdx.x >> 3;
  const int grp = m8 % NG;                                  // column group
  const int unit = (m8 / NG) * 8 + xcd;                     // (sequence, v-head)
  const int h = unit % a.hv;
  const int seq = unit / a.hv;
  if (seq >= a.num_seqs) return;
  int nseg, sbase;
  if (a.seqlen > 0) {
    nseg = nseg_of((a.seqlen + a.chunk - 1) / a.chunk, a.seg_len);
    sbase = seq * nseg;
  } else {
    sbase = a.seg_offsets[seq];
    nseg = a.seg_offsets[seq + 1] - sbase;
  }
  if (nseg < 3) return;
  const int last = nseg - 2;  // steps p = 1 .. last
  auto sptr = [&](int p) { return a.seg_state + ((long)(sbase + p) * a.hv + h) * DK * DV; };

  if (wave >= CW * RS) {
    const int lt = tid - 64 * CW * RS;
    struct Set {
      u32x4 pf[PV];
      f32x4 bf[BV];
    };
    auto load = [&](int p, Set& r) {  // Phi_p and B_p (held in S_start[p+1])
      const u32x4* ph = reinterpret_cast<const u32x4*>(a.seg_phi + ((long)(sbase + p) * a.hv + h) * DK * DK);
#pragma unroll
      for (int i = 0; i < PV; i++) r.pf[i] = ph[lt + LT * i];
      const float* b = sptr(p + 1);
#pragma unroll
      for (int i = 0; i < BV; i++) {
        const int w = lt + LT * i, u = w / (64 * CW), t = (w / 64) % CW, l = w % 64;
        r.bf[i] = *reinterpret_cast<const f32x4*>(b + state_frag<DV>(u, CW * grp + t, l));
      }
    };
    auto put = [&](int p, Set& r) {
#pragma unroll
      for (int i = 0; i < PV; i++) phl[p % NS][lt + LT * i] = r.pf[i];
#pragma unroll
      for (int i = 0; i < BV; i++) bl[p % NS][lt + LT * i] = r.bf[i];
    };
    // step p's data goes to ring slot p % NS just before barrier p; the
    // compute waves read it after that barrier
    Set r[NS];
#pragma unroll
    for (int q = 0; q < NS; q++)
      if (1 + q <= last) load(1 + q, r[q]);
    for (int p0 = 1; p0 <= last; p0 += NS) {
#pragma unroll
      for (int q = 0; q < NS; q++) {
        const int p = p0 + q;
        if (p <= last) {
          put(p, r[q]);
          if (p + NS <= last) load(p + NS, r[q]);
          lds_barrier();
        }
      }
    }
    return;
  }

  const int ct = wave / RS, rs = wave % RS;  // column tile, row share
  const int jt = CW * grp + ct;
  f32x4 S[NDT];
  {
    const float* s1 = sptr(1);
#pragma unroll
    for (int u = 0; u < NDT; u++) S[u] = *reinterpret_cast<const f32x4*>(s1 + state_frag<DV>(u, jt, lane));
  }
  for (int p = 1; p <= last; p++) {
    lds_barrier();
    const int b = p % NS;
    if constexpr (RS > 1) {
      // the other shares' rows of S_p, written at step p - 1
      if (p > 1) {
#pragma unroll
        for (int u = 0; u < NDT; u++)
          if (u / UPR != rs) S[u] = sx[(((p & 1) * CW + ct) * NDT + u) * 64 + lane];
      }
    }
    f32x4 acc[UPR];
#pragma unroll
    for (int i = 0; i < UPR; i++) acc[i] = bl[b][((rs * UPR + i) * CW + ct) * 64 + lane];
#pragma unroll
    for (int m = 0; m < KS; m++) {
      const bf16x8 zb = frag_acc(S[2 * m], S[2 * m + 1]);
#pragma unroll
      for (int i = 0; i < UPR; i++)
        acc[i] = mfma16(__builtin_bit_cast(bf16x8, phl[b][((rs * UPR + i) * KS + m) * 64 + lane]), zb, acc[i]);
    }
    float* dst = sptr(p + 1);
#pragma unroll
    for (int i = 0; i < UPR; i++) {
      const int u = rs * UPR + i;
      S[u] = acc[i];
      *reinterpret_cast<f32x4*>(dst + state_frag<DV>(u, jt, lane)) = acc[i];
      if constexpr (RS > 1) sx[((((p + 1) & 1) * CW + ct) * NDT + u) * 64 + lane] = acc[i];
    }
  }
}

// ------------------------------------------------------------------ pass 2
// Eight waves: 0..3 carry the state (NCT column tiles each) and write the
// outputs, 4..7 stage the chunks and form each chunk's P while the carry
// works up to its last product, which waits for P at a second barrier.  The staging registers live only
// in the staging waves, so the carry keeps its accumulators in VGPRs.
//
// NORM: the gated RMS norm is applied to o before it is written (the
// oxydllm notes, "Performance": the gated norm runs fused): each (token,
// v-head) row becomes y = w * o / sqrt(mean(o^2) + eps) * silu(z), with o
// rounded to bf16 first, as the separate kernel reads it.  A row's 128
// columns belong to the four carry waves, so each wave adds up the squares
// of its columns per token and leaves them in LDS (double-buffered by chunk
// parity); the next chunk's first barrier publishes them, and the rows are
// finished while the carry waves wait for the next chunk's P.  A chunk's o
// stays in registers (bf16) until then; the staging waves load its gate
// rows a chunk ahead and leave them in the chunk's V buffer, which the
// carry no longer reads after the chunk's P barrier.
template <int C, int DK, int DV, int NCW, bool NORM>
__global__ void __launch_bounds__(64 * (NCW + 4)) k_seg_pass2(ScanArgs a) {
  typedef SegSmem<C, DK, DV, true> SM;
  constexpr int NDT = DK / 16;
  constexpr int NCT = DV / (16 * NCW);  // state column tiles per carry wave
  static_assert(NCT * 16 * NCW == DV, "state columns must split over the carry waves");
  __shared__ SM sm;
  __shared__ float nss[NORM ? 2 * NCW * C : 1];  // [parity][carry wave][token]: row sums of o^2
  __shared__ __align__(16) float nwl[NORM ? DV : 4];  // the norm weight, read by the carry waves from LDS
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int c16 = lane & 15, r4 = 4 * (lane >> 4);
  int n, hk, h;
  block_unit(a, n, hk, h);
  const Seg sg = seg_of(a, C, n);
  if (sg.seq < 0) return;
  const int nch_seq = (sg.s1 - sg.s0 + C - 1) / C;
  const int ch0 = sg.p * a.seg_len;
  const int nch = max(0, min(a.seg_len, nch_seq - ch0));

  if (wave >= NCW) {
    // staging: chunk i+1 is written to LDS and chunk i+2 requested while
    // the carry waves work on chunk i
    Stager<C, DK, DV, true, 256> st;
    init_stager(st, a, sg, hk, h, tid - 64 * NCW);
    if constexpr (NORM)
      st.setup_z(reinterpret_cast<const uint16_t*>(a.norm_z) + (long)sg.s0 * a.stride_z + (long)h * DV, a.stride_z);
    if (nch > 0) {
      st.load(ch0);
      st.setup_tt(sm);
      st.store(sm, 0);
      if (nch > 1) st.load(ch0 + 1);
      if constexpr (NORM) st.zload(ch0, a.stride_z);
    }
    for (int i = 0; i < nch; i++) {
      lds_barrier();
      compute_p<C, DK, DV, 4>(sm, i & 1, wave - NCW, lane);
      lds_barrier();  // P ready for the carry's last product
      // NORM: chunk i's gate rows into its V buffer, which the carry no
      // longer reads; the carry waves use them after the next barrier
      if constexpr (NORM) st.zstore(sm, i & 1);
      if (i + 1 < nch) st.store(sm, (i + 1) & 1);
      if (i + 2 < nch) st.load(ch0 + i + 2);
      if constexpr (NORM) {
        if (i + 1 < nch) st.zload(ch0 + i + 1, a.stride_z);
      }
    }
    if constexpr (NORM) {
      if (nch > 0) lds_barrier();  // publishes the last chunk's row sums and gate rows
    }
    return;
  }

  int vcol[NCT];
  f32x4 Z[NDT][NCT];
  const float* sin = a.state_in ? a.state_in + ((long)sg.seq * a.hv + h) * DK * DV : nullptr;
  const float* sws = a.seg_state + ((long)(sg.sbase + sg.p) * a.hv + h) * DK * DV;
#pragma unroll
  for (int j = 0; j < NCT; j++) vcol[j] = 16 * (wave * NCT + j);
  // The start state: the branches enclose whole loops, so that each issues
  // all its loads before the first wait (a branch around each load makes
  // the compiler drain the loads in flight where it rejoins: one memory
  // round trip per tile).
  if (sg.nseg > 1) {
#pragma unroll
    for (int j = 0; j < NCT; j++)
#pragma unroll
      for (int u = 0; u < NDT; u++)
        Z[u][j] = *reinterpret_cast<const f32x4*>(sws + state_frag<DV>(u, wave * NCT + j, lane));
  } else if (sin) {
#pragma unroll
    for (int j = 0; j < NCT; j++)
#pragma unroll
      for (int u = 0; u < NDT; u++)
#pragma unroll
        for (int e = 0; e < 4; e++) Z[u][j][e] = sin[(long)(16 * u + r4 + e) * DV + vcol[j] + c16];
  } else {
#pragma unroll
    for (int j = 0; j < NCT; j++)
#pragma unroll
      for (int u = 0; u < NDT; u++) Z[u][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const long orow = (long)a.hv * DV;
  uint16_t* obase = reinterpret_cast<uint16_t*>(a.o) + (long)sg.s0 * orow + (long)h * DV;
  // o (or y) rows of chunk i of this segment, NCT tiles of bf16 in the
  // output layout: lane (c16, g) holds columns 4g..4g+3 of tile j for token
  // 16t + c16
  auto store_rows = [&](int i, const u32x2 (&rows)[NCT][C / 16]) {
    const int cs = (ch0 + i) * C;
    const int clen = min(C, sg.s1 - sg.s0 - cs);
    uint16_t* oc = obase + (long)cs * orow;
#pragma unroll
    for (int t = 0; t < C / 16; t++) {
      const int tok = 16 * t + c16;
      if constexpr (NCT == 2) {
        // lanes g and g^1 (16 apart) trade halves so that each writes 8
        // adjacent columns: even g the first tile, odd g the second.  The
        // row swap (odd 16-lane rows of the first operand with even rows of
        // the second) leaves every lane exactly its 8 columns, in order,
        // with no trip through the LDS.
        const bool ev = ((lane >> 4) & 1) == 0;
        const auto s0 = __builtin_amdgcn_permlane16_swap(rows[0][t][0], rows[1][t][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(rows[0][t][1], rows[1][t][1], false, false);
        const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
        const int col = ev ? vcol[0] + r4 : vcol[1] + r4 - 4;
        if (tok < clen) *reinterpret_cast<u32x4*>(oc + (long)tok * orow + col) = w;
      } else if (tok < clen) {
#pragma unroll
        for (int j = 0; j < NCT; j++) *reinterpret_cast<u32x2*>(oc + (long)tok * orow + vcol[j] + r4) = rows[j][t];
      }
    }
  };
  u32x2 ob[NCT][C / 16];
  if constexpr (!NORM) {
    for (int i = 0; i < nch; i++) {
      lds_barrier();
      carry_chunk<C, DK, DV, NCT, true>(sm, i & 1, Z, vcol, lane, ob, [] { lds_barrier(); });
      store_rows(i, ob);
    }
  } else {
    // the fused gated norm (see above); the previous chunk's o in obp.  The
    // weights are read from LDS where they are used: held in registers
    // across the carry they made the kernel spill, and every spill reload
    // waited for all the o stores in flight (one load counter, in order).
    u32x2 obp[NCT][C / 16];
    for (int c = tid; c < DV; c += 64 * NCW) nwl[c] = a.norm_w[c];  // published by the loop's first barrier
    // this wave's part of each row's sum of squares -> LDS slot of the parity
    auto row_sums = [&](int i) {
#pragma unroll
      for (int t = 0; t < C / 16; t++) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NCT; j++) {
          const f32x4 o4 = bf4_to_f32(ob[j][t]);
#pragma unroll
          for (int e = 0; e < 4; e++) ss += o4[e] * o4[e];
        }
        ss = add_lane_xor32(add_lane_xor16(ss));
        if (lane < 16) nss[((i & 1) * NCW + wave) * C + 16 * t + c16] = ss;
      }
    };
    // y of chunk i from obp, the published row sums and the gate rows the
    // staging waves left in the chunk's V buffer; y overwrites obp
    auto finish = [&](int i) {
      f32x4 wn[NCT];
#pragma unroll
      for (int j = 0; j < NCT; j++) wn[j] = *reinterpret_cast<const f32x4*>(&nwl[vcol[j] + r4]);
#pragma unroll
      for (int t = 0; t < C / 16; t++) {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < NCW; w++) ss += nss[((i & 1) * NCW + w) * C + 16 * t + c16];
        const float inv_rms = 1.0f / sqrtf(ss * (1.0f / DV) + a.norm_eps);
#pragma unroll
        for (int j = 0; j < NCT; j++) {
          const f32x4 o4 = bf4_to_f32(obp[j][t]);
          const f32x4 z4 = bf4_to_f32(*reinterpret_cast<const u32x2*>(&sm.v[i & 1][16 * t + c16][vcol[j] + r4]));
          f32x4 y;
#pragma unroll
          for (int e = 0; e < 4; e++)
            y[e] = wn[j][e] * o4[e] * inv_rms *
                   (z4[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z4[e] * 1.44269504088896341f)));
          obp[j][t] = pack4_bf16(y);
        }
      }
      store_rows(i, obp);
    };
    for (int i = 0; i < nch; i++) {
      lds_barrier();  // also publishes chunk i-1's row sums
      carry_chunk<C, DK, DV, NCT, true>(sm, i & 1, Z, vcol, lane, ob, [&] {
        // in the wait for P: the previous chunk's rows are finished (its
        // gate rows come from LDS; only its o stays live across the carry)
        if (i > 0) finish(i - 1);
        lds_barrier();
      });
      row_sums(i);
#pragma unroll
      for (int j = 0; j < NCT; j++)
#pragma unroll
        for (int t = 0; t < C / 16; t++) obp[j][t] = ob[j][t];
    }
    if (nch > 0) {
      lds_barrier();
      finish(nch - 1);
    }
  }

  if (sg.p == sg.nseg - 1 && a.state_out) {
    float* so = a.state_out + ((long)sg.seq * a.hv + h) * DK * DV;
#pragma unroll
    for (int j = 0; j < NCT; j++)
#pragma unroll
      for (int u = 0; u < NDT; u++)
#pragma unroll
        for (int e = 0; e < 4; e++) so[(long)(16 * u + r4 + e) * DV + vcol[j] + c16] = Z[u][j][e];
  }
}

// State-column tiles (16 columns each) per combine workgroup, and the depth
// of its load ring (steps in flight ahead of the chain).
constexpr int kCombineWaves = 1;
constexpr int kCombineRowShares = 4;  // compute waves per column tile (2: 8.55 us, 8: 8.8 us, 4: 8.3 us)
constexpr int kCombineSlots = 2;
// Carry waves of pass 2 (each owns d_v / (16 kPass2CarryWaves) column tiles).
constexpr int kPass2CarryWaves = 4;

template <int C, int DK, int DV>
hipError_t launch_seg_t(const ScanArgs& a, hipStream_t s) {
  const int G = a.hv / a.hk;
  const int groups = a.max_segs * a.hk;
  const dim3 grid(8 * ((groups + 7) / 8) * G), block(256);
  constexpr int NW1 = (DV + DK) % 128 == 0 ? 8 : 4;  // pass 1: 32 (or 48) columns per wave
  hipLaunchKernelGGL((k_seg_pass1<C, DK, DV, NW1>), grid, dim3(64 * NW1), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    constexpr int CW = kCombineWaves, LW = 4, NG = DV / (16 * CW);
    constexpr int RS = kCombineRowShares <= DK / 16 ? kCombineRowShares : DK / 16;
    const int units = a.num_seqs * a.hv;
    hipLaunchKernelGGL((k_seg_combine<DK, DV, CW, RS, LW, kCombineSlots>), dim3(8 * ((units + 7) / 8) * NG),
                       dim3(64 * (CW * RS + LW)), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  constexpr int NCW = kPass2CarryWaves * 16 <= DV ? kPass2CarryWaves : DV / 16;
  if (a.norm_z) hipLaunchKernelGGL((k_seg_pass2<C, DK, DV, NCW, true>), grid, dim3(64 * (NCW + 4)), 0, s, a);
  else hipLaunchKernelGGL((k_seg_pass2<C, DK, DV, NCW, false>), grid, dim3(64 * (NCW + 4)), 0, s, a);
  return hipGetLastError();
}

template <int C>
hipError_t launch_seg_c(const ScanArgs& a, hipStream_t s) {
  if (a.dk == 128 && a.dv == 128) return launch_seg_t<C, 128, 128>(a, s);
  if (a.dk == 128 && a.dv == 64) return launch_seg_t<C, 128, 64>(a, s);
  if (a.dk == 64 && a.dv == 128) return launch_seg_t<C, 64, 128>(a, s);
  if (a.dk == 64 && a.dv == 64) return launch_seg_t<C, 64, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool seg_path(const ScanArgs& a) {
  return a.dtype == 1 && (a.chunk == 32 || a.chunk == 64) && (a.dk == 64 || a.dk == 128) &&
         (a.dv == 64 || a.dv == 128);
}

hipError_t launch_seg(const ScanArgs& a, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  return a.chunk == 64 ? launch_seg_c<64>(a, s) : launch_seg_c<32>(a, s);
}

}  // namespace gdn
