// gfx950 (MI355X) kernels of the fused sparse-MLA attention step.
//
// The step [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose]: per token,
// per-head RMSNorm and RoPE on q, a gather of that token's own index rows from an
// E4M3 + UE8M0 latent pool (K = V, shared by all heads), softmax attention, inverse
// RoPE on the output and an E4M3 cast with UE8M0 block-32 scales.  Entries at or
// beyond topk_length are never read and -1 marks an empty slot [same page, Purpose,
// bug-fix bullet].
//
// Two main kernels compute the step:
//   smla_ws    the production shape (d = 512, E4M3 + UE8M0 pool, rope_dim 0 or 64): a
//              persistent grid of one 512-thread workgroup per compute unit walking the
//              work items (token, split), with QK and P.V waves specialized per SIMD and
//              one barrier per 64-entry tile (its own comment below has the details);
//   smla_main  every other shape: one workgroup per work item, described here.
// smla_combine (smla_main's splits, and the two-pool smla_nv's at rotary widths other
// than 0 and 64) and smla_combine_lm4 / smla_combine_lm1 (smla_ws's splits, stored in
// the P.V waves' register order, and smla_nv's in the same format; 4 or 1 float4 slots
// per thread) merge the splits of a token when a call is split.
//
// smla_main: one 512-thread workgroup (8 wave64, two per SIMD) per token, or per token
// split when few tokens are in flight.
//   prologue   one thread per (head, 32-dim block): q -> RMSNorm -> RoPE (angles in
//              fp64) -> times sm_scale*log2(e).  For the E4M3 pool q is split into two
//              E4M3 terms (hi + lo) with their own UE8M0 scales per 32 dims (about 8
//              significant bits); each wave keeps the fragments of its 32 heads x 256
//              dims in VGPRs for the whole token.
//   per tile of 64 index entries (row ids prefetched two tiles ahead, raw rows one
//   tile ahead by LDS DMA into a double buffer):
//     QK^T     wave (a, c, d) computes the partial S^T[32 rows of half c][32 heads of
//              group a] over dim half d with v_mfma_scale_f32_32x32x64_f8f6f4: K is the
//              raw E4M3 row data with its UE8M0 block scales as the MFMA's A scales, q
//              the hi / lo terms as B -- no dequantization of K at all.  (bf16 pool:
//              v_mfma_f32_32x32x16_bf16.)  The two dim halves meet through LDS.
//     V tile   the same raw rows are dequantized once (v_cvt_scalef32_pk_bf16_fp8,
//              exact) into a transposed bf16 tile Vt[dim][slot]; rows are stored in a
//              slot order that makes both the transpose's reads and writes and the
//              P.V reads bank-conflict free.  The two waves of a SIMD run QK and the
//              V tile in opposite orders so that MFMA and VALU work overlap.
//     softmax  per-head tile max shared through LDS by the two row halves; the running
//              max is raised only when the tile max exceeds it by 2^8 (lazy rescale);
//              P is rounded to bf16 (v_cvt_pk_bf16_f32) and stored [head][slot].
//     P.V      wave w owns output dims [64w, 64w + 64) for all 64 heads
//              (v_mfma_f32_32x32x16_bf16, accumulators in VGPRs).
//   epilogue   o = acc / l -> LDS -> inverse RoPE -> per-32 amax -> UE8M0 exponent
//              (integer test against 448 * 2^(e-127)) -> E4M3 by the scaled RNE convert.
//   split mode each workgroup writes (acc, m, l) for its share of the tiles; a second
//              kernel combines the splits of each (token, head) in split order and runs
//              the same epilogue.
#include <hip/hip_runtime.h>
#include <math.h>

#include <cmath>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "smla_internal.h"

#include "smla_device.h"

namespace smla {
namespace {

template <int D, int EB>
__global__ __launch_bounds__(NTHREADS, 1) void smla_main(KArgs a) {
  using C = Cfg<D, EB>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
  float* maxx = reinterpret_cast<float*>(smem + C::OFF_MAXX);
  float* alpha_l = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
  int* flag_l = reinterpret_cast<int*>(smem + C::OFF_FLAG);
  float* lsum = reinterpret_cast<float*>(smem + C::OFF_LSUM);
  float* cs = reinterpret_cast<float*>(smem + C::OFF_COS);
  float* sn = reinterpret_cast<float*>(smem + C::OFF_SIN);
  unsigned char* vt_l = smem + C::OFF_VT;
  unsigned char* p_l = smem + C::OFF_P;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int lrow = lane & 31, lhalf = lane >> 5;
  // QK roles: head group qa, row half qc, dim half qd.  Waves w and w + 4 share a SIMD
  // and hold the two dim halves of the same S block.
  const int qa = w & 1, qc = (w >> 1) & 1, qd = w >> 2;
  const int ns = a.num_splits;
  const int t = blockIdx.x / ns, split = blockIdx.x % ns;
  const int pos = a.positions[t];

  // ---------------- tile range of this workgroup
  const int lraw = a.topk_length[t];
  const int lcap = lraw < 0 ? 0 : (lraw > a.topk ? a.topk : lraw);
  const int ntile = (lcap + T - 1) / T;
  const int tb = split * a.tiles_per_split;
  const int te_raw = tb + a.tiles_per_split;
  const int te = te_raw < ntile ? te_raw : ntile;
  const int32_t* idx_t = a.indices + (size_t)t * a.topk;

  // Index entry tile*64 + lane, fetched one or two tiles before it is used.  The load
  // is unconditional (clamped into the row) and its value is only looked at after the
  // tile loop's own vmcnt(0): a compiler-generated wait for it would also wait for the
  // row DMA issued in the same tile.
  auto fetch_id = [&](int tile) -> int {
    const int j = tile * T + lane;
    return a.topk > 0 ? idx_t[j < a.topk ? j : a.topk - 1] : -1;
  };
  // the id if entry tile*64 + lane is read, else -1 (beyond the length, a sentinel, or
  // outside [0, n_rows))
  auto valid_id = [&](int tile, int raw) -> int {
    const int j = tile * T + lane;
    return (tile < te && j < lcap && raw >= 0 && (long long)raw < a.n_rows) ? raw : -1;
  };

  // Enqueue the LDS DMA of one tile's rows (and scales) into raw / sc.  Rows that are not
  // read come in as zeros (an out-of-range offset): the QK masks them and P is zero.
  const __amdgpu_buffer_rsrc_t pool_rs = buf_rsrc(a.pool, (uint32_t)(a.n_rows * C::RB));
  const __amdgpu_buffer_rsrc_t scale_rs = buf_rsrc(a.scales, (uint32_t)(a.n_rows * C::NSB));
  auto issue_tile = [&](int id_vec, unsigned char* raw, unsigned char* sc, int lane) {
    constexpr int GPW = (T / C::G) / NWAVES;  // DMA groups per wave
    constexpr int WPR = C::NSB / 4;           // 4-byte scale words per row
    // all row ids first (one round of cross-lane reads), then the DMA instructions
    int id[GPW + 1];
#pragma unroll
    for (int k = 0; k < GPW; ++k) id[k] = __shfl(id_vec, C::G * (GPW * w + k) + lane % C::G);
    const int f = 64 * w + lane;
    if constexpr (EB == 1) id[GPW] = __shfl(id_vec, (f / WPR) & 63);
#pragma unroll
    for (int k = 0; k < GPW; ++k) {
      const int gi = GPW * w + k;
      const int chunk = lane / C::G;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(raw + gi * C::GS));
      dma16(id[k] >= 0 ? (uint32_t)id[k] * C::RB + 16 * chunk : kNoRow, pool_rs, dst);
    }
    if constexpr (EB == 1) {
      if (w < WPR) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(sc + 256 * w));
        dma4(id[GPW] >= 0 ? (uint32_t)id[GPW] * C::NSB + 4 * (f % WPR) : kNoRow, scale_rs, dst);
      }
    }
  };

  // ---------------- prologue
  // The first tile's row DMA is issued as soon as the q loads are in flight; the q tile
  // sits above the raw tiles.  A rotary slice too long for the staging area there is
  // staged at offset 0 instead, and the DMA waits for the prologue.
  int raw_cur = fetch_id(tb);
  int raw_next = fetch_id(tb + 1);
  // the rotary staging (none for rope_dim 64) sits above the raw tiles when it fits below
  // the small area
  const bool early = a.rope_dim == 64 || C::RAW_END + HP * (a.rope_dim + 4) * 4 <= C::BIG;
  float* ystage = reinterpret_cast<float*>(smem + (early ? C::RAW_END : 0));
  q_prologue<C>(smem, t, pos, a, cs, sn, ystage, [&]() {
    if (early && tb < te) issue_tile(valid_id(tb, raw_cur), smem + C::OFF_RAW0, smem + C::OFF_SC0, lane);
  });
  __syncthreads();
  // Q fragments (B operand of S^T = K Q^T) of the 32 heads of group qa over dim half qd.
  //   E4M3 pool: k-step ks covers dims [64ks, 64ks+64); lane half h holds dims
  //   64ks + 16h + [0,16) and 64ks + 32 + 16h + [0,16) of its head (the 32x32x64 f8
  //   operand layout); the UE8M0 scale of block 2ks + h sits in byte ks - KSW8*qd of
  //   qs8[term].
  //   bf16 pool: step ks, lane half h holds dims 16ks + 8h + [0, 8).
  i32x8 qf8[2][(EB == 1) ? C::KSW8 : 1];
  uint32_t qs8[2];
  bf16x8 qbf[(EB == 2) ? C::KSW : 1];
  const uint32_t hsel = lhalf ? 0x07050301u : 0x06040200u;  // bytes 2j + h of 8
  if constexpr (EB == 1) {
#pragma unroll
    for (int term = 0; term < 2; ++term) {
      const unsigned char* qrow = smem + C::OFF_Q + (term * HP + 32 * qa + lrow) * C::QS8 + 16 * lhalf;
#pragma unroll
      for (int j = 0; j < C::KSW8; ++j) {
        const int ks = C::KSW8 * qd + j;
        const uint4 lo = *reinterpret_cast<const uint4*>(qrow + 64 * ks);
        const uint4 hi = *reinterpret_cast<const uint4*>(qrow + 64 * ks + 32);
        qf8[term][j] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                               (int)hi.w};
      }
      qs8[term] = scale_word<C>(smem + C::OFF_Q + C::OFF_QSC + (term * HP + 32 * qa + lrow) * C::NSB, qd, hsel);
    }
  } else {
    const unsigned short* qrow = reinterpret_cast<const unsigned short*>(smem + C::OFF_Q) + (32 * qa + lrow) * C::QS;
#pragma unroll
    for (int j = 0; j < C::KSW; ++j)
      qbf[j] = *reinterpret_cast<const bf16x8*>(qrow + 16 * (C::KSW * qd + j) + 8 * lhalf);
  }
  if (!early) {
    __syncthreads();  // staging (at offset 0) read before the DMA lands there
    if (tb < te) issue_tile(valid_id(tb, raw_cur), smem + C::OFF_RAW0, smem + C::OFF_SC0, lane);
  }
  f32x16 acc[2][C::NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's first-tile DMA has landed

  auto tile_step = [&](int tile, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    unsigned char* raw_l = smem + (BUF == 0 ? C::OFF_RAW0 : C::OFF_RAW1);
    unsigned char* sc_l = smem + (BUF == 0 ? C::OFF_SC0 : C::OFF_SC1);
    unsigned char* raw_n = smem + (BUF == 0 ? C::OFF_RAW1 : C::OFF_RAW0);
    unsigned char* sc_n = smem + (BUF == 0 ? C::OFF_SC1 : C::OFF_SC0);
    __syncthreads();  // B1: this tile's rows visible; Vt / P / partial S free
    // lane-dependent values recomputed per tile (keeps them out of the live set)
    const int tid = (int)threadIdx.x + opaque_zero();
    const int lane = tid & 63, lrow = lane & 31, lhalf = lane >> 5;
    const uint32_t hsel = lhalf ? 0x07050301u : 0x06040200u;
    const int id_cur = valid_id(tile, raw_cur);
    const unsigned long long mask = __ballot(id_cur >= 0);
    const int id_next = valid_id(tile + 1, raw_next);
    const int raw_next2 = fetch_id(tile + 2);
#ifdef SMLA_DEBUG_CHECKS
    if (w == 0)
      debug_flag_tile(a.sched, a.n_rows, tile < te && tile * T + lane < lcap, raw_cur, id_cur >= 0,
                      EB == 1 ? sc_l + C::NSB * lane : nullptr, C::NSB);
#endif

    // ---- QK^T: partial S^T[32 rows of half qc][32 heads of group qa] over dim half qd
    f32x16 s;
    auto qk = [&]() {
      const int r = 32 * qc + lrow;
      if constexpr (EB == 1) {
        const uint32_t ksc = scale_word<C>(sc_l + r * C::NSB, qd, hsel);
        i32x8 A[C::KSW8];
#pragma unroll
        for (int j = 0; j < C::KSW8; ++j) {
          const int ks = C::KSW8 * qd + j;
          const uint4 lo = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(r, 4 * ks + lhalf));
          const uint4 hi = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(r, 4 * ks + 2 + lhalf));
          A[j] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        qk_block<C::KSW8, true>(s, A, qf8[0], qf8[1], ksc, qs8[0], qs8[1]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int j = 0; j < C::KSW; ++j) {
          const bf16x8 A =
              *reinterpret_cast<const bf16x8*>(raw_l + raw_off<C>(r, 2 * (C::KSW * qd + j) + lhalf));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qbf[j], s, 0, 0, 0);
        }
      }
    };

    // ---- V tile: raw rows -> Vt[dim][slot] bf16.  A block is the 4 rows 8q + p + 2k
    // (k = 0..3, slots 8q + 4p + k) of one 16-byte chunk c.
    auto vtrans = [&]() {
      constexpr int NBLK = (T / 4) * C::NCH;
      if constexpr (C::NCH == 32 && C::G == 2 && EB == 1) {
        // one block per thread.  An 8-lane group covers 4 consecutive chunks x both
        // parities, so each read step touches 8 distinct bank slots and each write step
        // 16 distinct 8-byte slots.  Rows 8q + p + 2k sit in group 4q + k at parity p.
        static_assert(NBLK == NTHREADS, "one V block per thread");
        const int u = lane & 7, g8 = lane >> 3;
        const int c = 4 * g8 + (u >> 1), p = u & 1, q = w;
        const unsigned char* rbase = raw_l + 4 * q * C::GS + 16 * (2 * c + p);
        const unsigned char* sbase = sc_l + (8 * q + p) * C::NSB + (c >> 1);
        uint4 rw[4];
        uint32_t sb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // all loads first, one wait
          rw[k] = *reinterpret_cast<const uint4*>(rbase + k * C::GS);
          sb[k] = sbase[2 * k * C::NSB];
        }
        uint32_t pk[4][8];  // [k][element pair]
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float sc = ue8m0_f32(sb[k]);
          pk[k][0] = cvt_lo(rw[k].x, sc); pk[k][1] = cvt_hi(rw[k].x, sc);
          pk[k][2] = cvt_lo(rw[k].y, sc); pk[k][3] = cvt_hi(rw[k].y, sc);
          pk[k][4] = cvt_lo(rw[k].z, sc); pk[k][5] = cvt_hi(rw[k].z, sc);
          pk[k][6] = cvt_lo(rw[k].w, sc); pk[k][7] = cvt_hi(rw[k].w, sc);
        }
        // dim n = 16c + e: swz(n) = (e & 7) ^ (e >> 3) ^ K0 with K0 = (2c ^ (c >> 2)) & 7,
        // so the 16-byte slot is (q ^ K0) ^ E(e), E(e) = (e & 7) ^ (e >> 3).  In write
        // step e, lanes with f = 1 (8-lane groups 2, 3 of each half wave) write element
        // e ^ 1 instead: dim rows of both parities are written at once, so a half wave's
        // 256 bytes cover all 64 banks.  (f only flips bit 0 of the element: the register
        // pair e >> 1 stays the same, the byte selector and the row change.)
        const int f = (g8 >> 1) & 1;
        const int q0 = q ^ ((2 * c ^ (c >> 2)) & 7) ^ f;
        const uint32_t sel_even = f ? 0x07060302u : 0x05040100u;  // element e ^ f, e even
        const uint32_t sel_odd = f ? 0x05040100u : 0x07060302u;   // e odd
        unsigned char* wb_even = vt_l + 2048 * c + 8 * p + 128 * f;   // row 16c + (e ^ f)
        unsigned char* wb_odd = vt_l + 2048 * c + 8 * p - 128 * f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int k = e >> 1;
          const uint32_t sel = (e & 1) ? sel_odd : sel_even;
          const uint2 o = make_uint2(__builtin_amdgcn_perm(pk[1][k], pk[0][k], sel),
                                     __builtin_amdgcn_perm(pk[3][k], pk[2][k], sel));
          const int E = (e & 7) ^ (e >> 3);
          *reinterpret_cast<uint2*>(((e & 1) ? wb_odd : wb_even) + 128 * e + 16 * (q0 ^ E)) = o;
        }
      } else {
#pragma unroll
        for (int bb0 = 0; bb0 < NBLK; bb0 += NTHREADS) {
          const int bb = bb0 + tid;
          if (NBLK % NTHREADS != 0 && bb >= NBLK) break;
          const int p = bb & 1, c = (bb >> 1) % C::NCH, q = (bb >> 1) / C::NCH;
          uint32_t pk[4][C::CE / 2];  // [k][element pair]
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int row = 8 * q + p + 2 * k;
            const uint4 rw = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(row, c));
            if constexpr (EB == 1) {
              const float sc = ue8m0_f32(sc_l[row * C::NSB + (c >> 1)]);
              pk[k][0] = cvt_lo(rw.x, sc); pk[k][1] = cvt_hi(rw.x, sc);
              pk[k][2] = cvt_lo(rw.y, sc); pk[k][3] = cvt_hi(rw.y, sc);
              pk[k][4] = cvt_lo(rw.z, sc); pk[k][5] = cvt_hi(rw.z, sc);
              pk[k][6] = cvt_lo(rw.w, sc); pk[k][7] = cvt_hi(rw.w, sc);
            } else {
              pk[k][0] = rw.x; pk[k][1] = rw.y; pk[k][2] = rw.z; pk[k][3] = rw.w;
            }
          }
#pragma unroll
          for (int e = 0; e < C::CE; ++e) {
            const int k = e >> 1;
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const uint2 o = make_uint2(__builtin_amdgcn_perm(pk[1][k], pk[0][k], sel),
                                       __builtin_amdgcn_perm(pk[3][k], pk[2][k], sel));
            const int n = C::CE * c + e;
            *reinterpret_cast<uint2*>(vt_l + n * 128 + 16 * (q ^ swz(n)) + 8 * p) = o;
          }
        }
      }
    };

    // The two waves of a SIMD run the halves in opposite order: one issues MFMAs while
    // the other converts.  The next tile's DMA goes out between the halves, after the
    // MFMA chain (qd 0) or the conversion (qd 1) has been issued.
    if (qd == 0) {
      qk();
      if (tile + 1 < te) issue_tile(id_next, raw_n, sc_n, lane);
      vtrans();
    } else {
      vtrans();
      if (tile + 1 < te) issue_tile(id_next, raw_n, sc_n, lane);
      qk();
    }
    if constexpr (EB == 1) qk_drain(s);  // the MFMA chain's results before any read of s

    // ---- partial S exchange: the dim-half-1 wave hands its partial to its partner
    float* sx = reinterpret_cast<float*>(smem + C::OFF_SX) + (w & 3) * 1024;
    if (qd == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(sx + 4 * (64 * j + lane)) = make_float4(s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]);
    }
    __syncthreads();  // B2a: partial S visible
    float mloc = -INFINITY;
    if (qd == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(sx + 4 * (64 * j + lane));
        s[4 * j] += v.x; s[4 * j + 1] += v.y; s[4 * j + 2] += v.z; s[4 * j + 3] += v.w;
      }
      // ---- softmax (part 1): tile max per head.  s is already in log2 units (q carries
      // sm_scale * log2(e)).  Row 32qc + 8g + 4h + j of value i = 4g + j is valid iff
      // its bit is set in the tile mask: the per-lane condition is built on the scalar
      // unit (lanes 0-31 take bit r, lanes 32-63 bit r + 4) and applied by one select.
      const uint32_t mw = (uint32_t)(mask >> (32 * qc));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + (i & 3);
        const unsigned long long lm = (((mw >> r) & 1u) ? 0x00000000FFFFFFFFull : 0ull) |
                                      (((mw >> (r + 4)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
        s[i] = __builtin_amdgcn_inverse_ballot_w64(lm) ? s[i] : -INFINITY;
        mloc = fmaxf(mloc, s[i]);
      }
      mloc = pair_max(mloc);
      if (lhalf == 0) maxx[qc * HP + 32 * qa + lrow] = mloc;
    }
    __syncthreads();  // B2: maxima exchanged

    // ---- softmax (part 2): running max (lazy), P in bf16 by slot, alpha
    if (qd == 0) {
      const float mt = fmaxf(mloc, maxx[(1 - qc) * HP + 32 * qa + lrow]);
      float mnew = m_run;
      if (mt > -INFINITY && (m_run == -INFINITY || mt > m_run + 8.0f)) mnew = mt;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
      // the accumulators need rescaling only where a finite running max was raised
      const bool raised = __any(m_run != -INFINITY && mnew != m_run);
      m_run = mnew;
      const float msafe = (mnew == -INFINITY) ? 0.f : mnew;  // masked scores are -inf: p = 0
      float p[16];
      float lp = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - msafe);
        lp += p[i];
      }
      l_run = l_run * alpha + lp;
      const int head = 32 * qa + lrow;
      unsigned char* prow = p_l + head * 128;
      const int sw = swz(head);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // rows 32qc + 8g + 4h + i -> slots 8(4qc + g) + 2h + {0, 1} (i = 0, 2) and
        // 8(4qc + g) + 4 + 2h + {0, 1} (i = 1, 3)
        const int q8 = 4 * qc + g;
        unsigned char* cbase = prow + 16 * (q8 ^ sw) + 4 * lhalf;
        *reinterpret_cast<uint32_t*>(cbase) = pack_bf16(p[4 * g + 0], p[4 * g + 2]);
        *reinterpret_cast<uint32_t*>(cbase + 8) = pack_bf16(p[4 * g + 1], p[4 * g + 3]);
      }
      if (qc == 0 && lhalf == 0) alpha_l[head] = alpha;
      if (qc == 0 && lane == 0) flag_l[qa] = raised ? 1 : 0;
    }
    __syncthreads();  // B3: P and alpha visible

    // ---- P.V: O[64 heads][dims of wave w]
    if (w < C::PVW) {
      const int2 fl = *reinterpret_cast<const int2*>(flag_l);
      if (__builtin_amdgcn_readfirstlane(fl.x | fl.y)) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 v4 = *reinterpret_cast<const float4*>(alpha_l + 32 * mb + 8 * g + 4 * lhalf);
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
              acc[mb][nb][4 * g + 0] *= v4.x;
              acc[mb][nb][4 * g + 1] *= v4.y;
              acc[mb][nb][4 * g + 2] *= v4.z;
              acc[mb][nb][4 * g + 3] *= v4.w;
            }
          }
      }
      const int d0 = C::DQ * w;
#pragma unroll
      for (int ks = 0; ks < T / 16; ++ks) {
        const int ch = 2 * ks + lhalf;
        bf16x8 A[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int h = 32 * mb + lrow;
          A[mb] = *reinterpret_cast<const bf16x8*>(p_l + h * 128 + 16 * (ch ^ swz(h)));
        }
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const int n = d0 + 32 * nb + lrow;
          const bf16x8 B = *reinterpret_cast<const bf16x8*>(vt_l + n * 128 + 16 * (ch ^ swz(n)));
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mb], B, acc[mb][nb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile's DMA from this wave landed
    raw_cur = raw_next;
    raw_next = raw_next2;
  };

  for (int tile = tb; tile < te; tile += 2) {
    tile_step(tile, std::integral_constant<int, 0>{});
    if (tile + 1 < te) tile_step(tile + 1, std::integral_constant<int, 1>{});
  }

  // ---------------- finish: l per head, then normalize + epilogue, or write partials
  if (qd == 0) {
    const float lw = pair_sum(l_run);
    if (lhalf == 0) lsum[qc * HP + 32 * qa + lrow] = lw;
    if (qc == 0 && lhalf == 0) maxx[32 * qa + lrow] = m_run;
  }
  __syncthreads();
  const int d0 = C::DQ * w;
  if (ns == 1) {
    float* o_l = reinterpret_cast<float*>(smem);
    if (w < C::PVW) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int h = 32 * mb + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          const float lt = lsum[h] + lsum[HP + h];
          const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) o_l[h * C::OS + d0 + 32 * nb + lrow] = acc[mb][nb][i] * inv;
        }
    }
    __syncthreads();
    epilogue<D, NTHREADS>(o_l, C::OS, a.h_q, 0, t, a, cs, sn);
  } else {
    float* part = a.ws + ((size_t)t * ns + split) * partial_floats_d(a.h_q, D);
    float* pm = part + (size_t)HP * D;
    float* pl = pm + HP;
    if (tid < a.h_q) {
      pm[tid] = maxx[tid];
      pl[tid] = lsum[tid] + lsum[HP + tid];
    }
    if (te > tb && w < C::PVW) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int h = 32 * mb + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          if (h < a.h_q) {
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) part[(size_t)h * D + d0 + 32 * nb + lrow] = acc[mb][nb][i];
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Persistent warp-specialized kernel for d = 512, rope_dim 0 or 64, E4M3 pool (the
// production shape).
//
// Each workgroup walks the work items (token, split) blockIdx.x, blockIdx.x + gridDim.x,
// ...  The eight waves split into two roles, one wave of each per SIMD:
//   QK waves (w = 0..3, head group qa = w & 1, row half qc = w >> 1) hold q for their
//     32 heads over all 512 dims in VGPRs and compute S^T[32 rows][32 heads] of a tile
//     with 16 scaled E4M3 MFMAs, then the softmax of that block.
//   P.V waves (w = 4..7) own output dims [128v, 128v + 128) for all 64 heads.  They take
//     V straight from the raw E4M3 rows: one scaled E4M3 MFMA of 32 rows x 64 dims against
//     an identity operand yields a 32 x 32 block of V dequantized exactly and transposed
//     (lane = dim, registers = slots), which, packed to bf16, is the A operand of the
//     P.V MFMAs; the P.V contraction visits the slots in that register order and the QK
//     waves store P in the same order (details at the P.V iteration below).  They also
//     issue all row DMA of the next tile.
// Iteration i: QK waves compute S and P of tile i, P.V waves P.V of tile i - 1 and the DMA
// of tile i + 1 (three raw tile buffers); one barrier per iteration.  The softmax is taken
// against the running max of the previous tiles: a QK wave flags its head group when its
// block max exceeds that max by more than 2^8.  The flags are read after the barrier; if
// any is set (always on the first tile), the QK waves merge the block maxima of both row
// halves, raise the running max, rewrite P from the scores they still hold and publish
// the accumulator rescale, and a second barrier lets the P.V waves go on.  The running
// max is therefore the same lazily raised max as in the generic kernel.
// Between items: the P.V waves run the epilogue of the finished item straight from their
// registers (their MFMAs produce O^T, so a head's 32-dim block sits in one lane pair),
// while the QK waves issue the next item's first tile DMA and run its q prologue into a
// q tile over the second and third raw tile buffers, from which they then load their
// fragments.
struct WsCfg {
  static constexpr int kD = 512, kEB = 1;
  static constexpr int D = kD;
  static constexpr int RB = D, NCH = D / 16, NSB = D / 32, G = 1024 / RB;
  static constexpr int GS = 1024 + 16 * G;
  static constexpr int RAW_BYTES = (T / G) * GS;
  static constexpr int SC_BYTES = T * NSB;
  static constexpr int P_BYTES = HP * T * 2;
  // three raw tiles (and their scale rows): tile i in buffer i mod 3, so that the QK waves
  // read tile i, the P.V waves tile i - 1 and the DMA fills tile i + 1 at once
  static constexpr int OFF_RAW0 = 0;
  static constexpr int OFF_RAW1 = RAW_BYTES;
  static constexpr int OFF_RAW2 = 2 * RAW_BYTES;
  static constexpr int OFF_SC0 = 3 * RAW_BYTES;
  static constexpr int OFF_SC1 = OFF_SC0 + SC_BYTES;
  static constexpr int OFF_SC2 = OFF_SC1 + SC_BYTES;
  static constexpr int OFF_P0 = align16(OFF_SC2 + SC_BYTES);
  static constexpr int OFF_P1 = OFF_P0 + P_BYTES;
  static constexpr int LOOP_END = OFF_P1 + P_BYTES;
  // between items: the q tile [2 terms][HP][512 B] (16-byte chunk c of head h stored at
  // c ^ (h & 15)) over raw tiles 1 and 2 (an item's first tile lands in tile 0), its UE8M0
  // scales [2][HP][16] in P0
  static constexpr int OFF_QT = OFF_RAW1;
  static constexpr int OFF_QSC = OFF_P0;
  // small area
  static constexpr int OFF_MAXX = LOOP_END;                // [2 tiles][2 row halves][HP]
  static constexpr int OFF_ALPHA = OFF_MAXX + 4 * HP * 4;  // [HP]
  static constexpr int OFF_LSUM = OFF_ALPHA + HP * 4;      // [2 row halves][HP]
  static constexpr int OFF_MFIN = OFF_LSUM + 2 * HP * 4;   // [HP]
  static constexpr int OFF_FLAG = OFF_MFIN + HP * 4;       // overflow [2 tiles][4], rescale [2]
  // per wave: cos[32], sin[32], then the rotary blocks' q factors A14, B14, A15, B15 [32]
  static constexpr int OFF_ROPE = OFF_FLAG + 64;
  static constexpr int ROPE_FLOATS = 192;
  static constexpr int OFF_NW = OFF_ROPE + NWAVES * ROPE_FLOATS * 4;  // norm_w, block b at 36 b floats
  static constexpr int OFF_IFREQ = OFF_NW + (D / 32) * 36 * 4;  // theta^(-2i/r), i < 32, fp64
  static constexpr int OFF_ZERO = OFF_IFREQ + 32 * 8;             // 32 zeros
  static constexpr int SMEM = OFF_ZERO + 32 * 4;
  static_assert(G == 2 && NSB == 16, "layout written for 512-byte rows");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(2 * HP * 512 <= 2 * RAW_BYTES && 2 * HP * 16 <= P_BYTES, "item transition areas");
};

__global__ __launch_bounds__(NTHREADS, 1) void smla_ws(KArgs a) {
  using C = WsCfg;
  constexpr int D = C::D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
  float* maxx = reinterpret_cast<float*>(smem + C::OFF_MAXX);
  float* alpha_l = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
  int* flag_l = reinterpret_cast<int*>(smem + C::OFF_FLAG);
  float* lsum = reinterpret_cast<float*>(smem + C::OFF_LSUM);
  float* mfin = reinterpret_cast<float*>(smem + C::OFF_MFIN);
  // The kernel arguments used only between items, re-read from the kernarg segment
  // where they are needed (an opaque pointer), so that they are not held in registers
  // across the tile loops.
  auto karg = [&]() -> const __attribute__((address_space(4))) KArgs& {
    const __attribute__((address_space(4))) KArgs* p =
        (const __attribute__((address_space(4))) KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return *p;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int ns = a.num_splits;
  const int total = a.s_q * ns;
  const bool rot = a.rope_dim > 0;  // 0 or 64 on this path
  float* rtab = reinterpret_cast<float*>(smem + C::OFF_ROPE) + C::ROPE_FLOATS * w;  // this wave's table

  struct Item {
    int t, pos, lcap, tb, te, n;
  };
  auto info = [&](int slot) {
    Item I;
    const int item = a.order ? a.order[slot] : slot;
    I.t = item / ns;
    const int split = item % ns;
    I.pos = a.positions[I.t];
    const int lraw = a.topk_length[I.t];
    I.lcap = lraw < 0 ? 0 : (lraw > a.topk ? a.topk : lraw);
    const int ntile = (I.lcap + T - 1) / T;
    I.tb = split * a.tiles_per_split;
    const int te_raw = I.tb + a.tiles_per_split;
    I.te = te_raw < ntile ? te_raw : ntile;
    I.n = I.te > I.tb ? I.te - I.tb : 0;
    return I;
  };
  // Index entry tile*64 + lane, fetched before it is used (clamped into the row, read
  // through a range-checked buffer so that the load has no branch: with topk = 0 it reads
  // zero, which valid_id rejects); its value is only looked at after a wait that covers it.
  auto fetch_id = [&](const Item& I, int tile) -> int {
    const int j = tile * T + (((int)threadIdx.x + opaque_zero()) & 63);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.indices + (size_t)I.t * a.topk, (uint32_t)a.topk * 4u);
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(j < a.topk ? j : a.topk - 1) * 4u, 0, 0);
  };
  // the id if entry tile*64 + lane is read, else -1 (beyond the length, a sentinel, or
  // outside [0, n_rows))
  auto valid_id = [&](const Item& I, int tile, int raw) -> int {
    const int j = tile * T + (((int)threadIdx.x + opaque_zero()) & 63);
    return (tile < I.te && j < I.lcap && raw >= 0 && (long long)raw < a.n_rows) ? raw : -1;
  };
  const __amdgpu_buffer_rsrc_t pool_rs = buf_rsrc(a.pool, (uint32_t)(a.n_rows * C::RB));
  const __amdgpu_buffer_rsrc_t scale_rs = buf_rsrc(a.scales, (uint32_t)(a.n_rows * C::NSB));
  // One part of the LDS DMA of a tile, as if issued by wave vw: part k < 4 moves DMA group
  // 4vw + k (two rows, one 1 KB instruction; the rows' ids come from two lanes by
  // readlane), part 4 the scale rows of 16 ids (vw < 4, one shuffle).  Rows that are not
  // read come in as zeros.  counted: the compiler's own DMA loads (an item's first tile),
  // else the asm ones (the tile loop).
  auto dma_part = [&](int k, int vw, int id_vec, unsigned char* raw, unsigned char* sc, auto counted_c) {
    constexpr bool counted = decltype(counted_c)::value;
    const int lane = ((int)threadIdx.x + opaque_zero()) & 63;
    if (k < 4) {
      const int gi = 4 * vw + k;
      const int i0 = __builtin_amdgcn_readlane(id_vec, 2 * gi), i1 = __builtin_amdgcn_readlane(id_vec, 2 * gi + 1);
      const int id = (lane & 1) ? i1 : i0;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(raw + gi * C::GS));
      const uint32_t off = id >= 0 ? (uint32_t)id * C::RB + 16 * (lane >> 1) : kNoRow;
      if constexpr (counted) dma16c(off, pool_rs, dst); else dma16(off, pool_rs, dst);
    } else {
      const int f = 64 * vw + lane;
      const int id = __shfl(id_vec, (f / 4) & 63);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(sc + 256 * vw));
      const uint32_t off = id >= 0 ? (uint32_t)id * C::NSB + 4 * (f % 4) : kNoRow;
      if constexpr (counted) dma4c(off, scale_rs, dst); else dma4(off, scale_rs, dst);
    }
  };
  // tile i's raw rows and scales in buffer i mod 3 (i >= -1: the P.V waves ask for i - 1)
  auto raw_buf = [&](int i) {
    const int b = (i + 3) % 3;
    return smem + (b == 0 ? C::OFF_RAW0 : (b == 1 ? C::OFF_RAW1 : C::OFF_RAW2));
  };
  auto sc_buf = [&](int i) {
    const int b = (i + 3) % 3;
    return smem + (b == 0 ? C::OFF_SC0 : (b == 1 ? C::OFF_SC1 : C::OFF_SC2));
  };
  auto p_buf = [&](int i) { return smem + ((i & 1) ? C::OFF_P1 : C::OFF_P0); };

  // ---------------- q prologue of an item (in two steps)
  // With NU units per thread, thread tid handles block b = tid & 15 (32 dims) of heads
  // (tid >> 4) + (64 / NU) k, k < NU: a row of 16 lanes holds one head, whose sum of
  // squares is reduced with DPP.  Between items the QK waves run it alone (NU = 4); the
  // first item of a workgroup is split over all eight waves (NU = 2).
  auto q_load = [&](const Item& I, auto nu_c, uint4 (&x)[4][4]) {
    constexpr int NU = decltype(nu_c)::value;
    // lane-dependent values are recomputed in each phase (opaque_zero) instead of being
    // hoisted out of the item loop and kept live across it
    const int tid = (int)threadIdx.x + opaque_zero(), qb = tid & 15;
    const auto& K = karg();
    const int hq = K.h_q;
    // the token's rows as a range-checked buffer: heads >= h_q read as zeros without a
    // branch, so every load is issued unconditionally and waits on them can count
    const __amdgpu_buffer_rsrc_t qrs = buf_rsrc(K.q + (size_t)I.t * hq * D, (uint32_t)(hq * D * 2));
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int head = (tid >> 4) + (64 / NU) * k;
      const uint32_t off = (uint32_t)(head * D + 32 * qb) * 2u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 16u * j, 0, 0);
        x[k][j] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  };
  // cos / sin of angle pos * theta^(-2i/64), i < 32: the angle in fp64 (the inverse
  // frequencies are computed once per workgroup), reduced to [-pi, pi] (Cody-Waite with a
  // two-part 2*pi), then the hardware sine / cosine of the reduced angle in revolutions;
  // lane i of every wave computes entry i of the wave's own table: cos, sin, and the q
  // prologue's factors of the rotary pair (448 + i, 480 + i) with norm_w w folded in,
  // A14 = w448 c, B14 = -w480 s, A15 = w480 c, B15 = w448 s.
  const double* ifreq = reinterpret_cast<const double*>(smem + C::OFF_IFREQ);
  auto rope_tab = [&](const Item& I) {
    const int lane = ((int)threadIdx.x + opaque_zero()) & 63;
    if (rot && lane < 32) {
      constexpr double kInv2Pi = 0.15915494309189535, k2PiHi = 6.283185307179586, k2PiLo = 2.4492935982947064e-16;
      const double ang = (double)I.pos * ifreq[lane];
      const double nn = rint(ang * kInv2Pi);
      const double r = fma(-nn, k2PiLo, fma(-nn, k2PiHi, ang));
      const float rev = (float)(r * kInv2Pi);  // in [-1/2, 1/2]
      const float sv = __builtin_amdgcn_sinf(rev), cv = __builtin_amdgcn_cosf(rev);
      const float* nw = reinterpret_cast<const float*>(smem + C::OFF_NW);
      const float w0 = nw[36 * 14 + lane], w1 = nw[36 * 15 + lane];
      rtab[lane] = cv;
      rtab[32 + lane] = sv;
      rtab[64 + lane] = w0 * cv;
      rtab[96 + lane] = -(w1 * sv);
      rtab[128 + lane] = w1 * cv;
      rtab[160 + lane] = w0 * sv;
    }
  };
  // RMSNorm (f32), times sm_scale * log2(e) (the scores come out ready for exp2), RoPE on
  // dims 448..511, then two E4M3 terms with their own UE8M0 scales per block into the q
  // tile.  Norm and RoPE are one step per dim, y' = (A y + B y_partner) * qscale / rms: on
  // the rotary blocks 14 and 15 A and B are the wave table's norm_w * cos / sin products
  // (the partner, the same dim of the other block, comes through DPP), elsewhere A =
  // norm_w and B = 0, an exact identity, so the row needs no branch (a divergent one costs
  // the same issue slots plus copies of y at its join).
  auto q_units = [&](auto nu_c, const uint4 (&x)[4][4]) {
    constexpr int NU = decltype(nu_c)::value;
    const int tid = (int)threadIdx.x + opaque_zero(), qb = tid & 15;
    const auto& K = karg();
    const float qscale = K.sm_scale * 1.4426950408889634f, eps = K.rms_eps;
    const bool rl = rot && qb >= 14;
    const float* at = rl ? rtab + (qb == 14 ? 64 : 128) : reinterpret_cast<const float*>(smem + C::OFF_NW) + 36 * qb;
    const float* bt = rl ? rtab + (qb == 14 ? 96 : 160) : reinterpret_cast<const float*>(smem + C::OFF_ZERO);
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int head = (tid >> 4) + (64 / NU) * k;
      float y[32];
      // the sum of squares straight from the bf16 pairs (products exact in f32)
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t uu[4] = {x[k][j].x, x[k][j].y, x[k][j].z, x[k][j].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          y[8 * j + 2 * m] = bf16_f32(uu[m] & 0xFFFFu);
          y[8 * j + 2 * m + 1] = bf16_f32(uu[m] >> 16);
          const bf16x2 p = __builtin_bit_cast(bf16x2, uu[m]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
        }
      }
      // lane pairs i^1, i^2, then i <-> 7-i, i <-> 15-i: every lane of the row ends with
      // the same sum
      ss += dpp_f32<0xB1>(ss);
      ss += dpp_f32<0x4E>(ss);
      ss += dpp_f32<0x141>(ss);
      ss += dpp_f32<0x140>(ss);
      const float inv = qscale * __builtin_amdgcn_rsqf(ss / (float)D + eps);
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {
        const float4 a4 = *reinterpret_cast<const float4*>(at + 4 * q4);
        const float4 b4 = *reinterpret_cast<const float4*>(bt + 4 * q4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int e = 4 * q4 + m;
          // the partner (quad_perm [0,1,3,2]: lanes 14 <-> 15) times B: one v_mul with the
          // lane swap folded in, then one fma and the scale
          const float ps = dpp_perm_f32<0xB4>(y[e]) * bv[m];
          y[e] = __builtin_fmaf(y[e], av[m], ps) * inv;
        }
      }
      unsigned char* qt = smem + C::OFF_QT + head * 512;
      unsigned char* qsc = smem + C::OFF_QSC + head * 16 + qb;
      const int sw = head & 15;
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(y[e]));
      int eq = ue8m0_exp(amax);
#pragma unroll
      for (int term = 0; term < 2; ++term) {
        const float sc = ue8m0_f32((uint32_t)eq);
        uint32_t wd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          wd[j] = enc2(enc2(0u, y[4 * j], y[4 * j + 1], sc, false), y[4 * j + 2], y[4 * j + 3], sc, true);
        unsigned char* row = qt + term * HP * 512;
        *reinterpret_cast<uint4*>(row + 16 * ((2 * qb) ^ sw)) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        *reinterpret_cast<uint4*>(row + 16 * ((2 * qb + 1) ^ sw)) = make_uint4(wd[4], wd[5], wd[6], wd[7]);
        qsc[term * HP * 16] = (unsigned char)eq;
        if (term == 0) {
          // residual for the second term; an RNE E4M3 code is off by at most 16 of its
          // scale units, so 2^-4 of the first scale holds the residual unsaturated
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wd[j], sc, false);
            const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wd[j], sc, true);
            y[4 * j] -= d0[0];
            y[4 * j + 1] -= d0[1];
            y[4 * j + 2] -= d1[0];
            y[4 * j + 3] -= d1[1];
          }
          eq = eq >= 4 ? eq - 4 : 0;
        }
      }
    }
  };

  // Set-up shared by all waves, published by the first barrier of either branch (each
  // branch issues its first item's loads before its share of it): norm_w into LDS once
  // (block b at 36 b floats: the 16 lanes of a head read 16 distinct banks) and the
  // inverse frequencies theta^(-2i/r) in fp64.
  // The norm_w load goes out first so that its wait leaves the q loads in flight.
  float4 nw4;
  if (tid < D / 4) nw4 = reinterpret_cast<const float4*>(a.norm_w)[tid];
  auto setup = [&]() __attribute__((always_inline)) {
    if (tid < D / 4) *reinterpret_cast<float4*>(smem + C::OFF_NW + 4 * (36 * (tid / 8) + 4 * (tid % 8))) = nw4;
    if (rot && tid >= 448 && tid < 480) {
      const int i = tid - 448;
      reinterpret_cast<double*>(smem + C::OFF_IFREQ)[i] = exp2(-(2.0 * i / (double)a.rope_dim) * a.log2_theta);
    }
    if (tid >= 384 && tid < 416) reinterpret_cast<float*>(smem + C::OFF_ZERO)[tid - 384] = 0.f;
    __syncthreads();
  };

  if (w < 4) {
    // =============================== QK waves
    const int qa = w & 1, qc = w >> 1;
    int item = blockIdx.x;
    Item I = info(item);
    int raw_cur, raw_next;
    // an item's prologue (its first ids, id0, resolved and its q loads issued):
    // first-tile DMA (all of it, 9 instructions per wave), cos / sin table, q tile
    auto transition = [&](auto nu_c, uint4 (&x)[4][4], const int id0) {
      // the item after this one, from the workspace's counter: fetched first, published
      // (before B_A) last, so that waiting for it holds nothing up.  The address is made
      // opaque so that the compiler issues a plain returning atomic (a wave reduction
      // around it would wait for its result, and so for the q loads, on the spot).
      const bool leader = w == 0 && (((int)threadIdx.x + opaque_zero()) & 63) == 0;
      unsigned nx = 0;
      if (leader) nx = atomicAdd(a.sched + opaque_zero(), 1u);
      // the DMA is issued without a branch (an item without tiles moves zeros)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dma_part(k, w, id0, raw_buf(0), sc_buf(0), std::true_type{});
        dma_part(k, w + 4, id0, raw_buf(0), sc_buf(0), std::true_type{});
      }
      dma_part(4, w, id0, raw_buf(0), sc_buf(0), std::true_type{});
      rope_tab(I);
      // (the compiler's wait for q counts the counter fetch and the 9 DMA loads issued
      // after it, which stay in flight)
      q_units(nu_c, x);
      if (leader) flag_l[12] = (int)gridDim.x + (int)nx;
    };
    {
      raw_cur = fetch_id(I, I.tb);
      raw_next = fetch_id(I, I.tb + 1);
      uint4 x[4][4];
      q_load(I, std::integral_constant<int, 2>{}, x);
      setup();
      transition(std::integral_constant<int, 2>{}, x, valid_id(I, I.tb, raw_cur));
    }
    while (true) {
      __syncthreads();  // B_A: q tile complete
      const int next = __builtin_amdgcn_readfirstlane(flag_l[12]);
      const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
      const uint32_t hsel = lhalf ? 0x07050301u : 0x06040200u;
      // q of the 32 heads of group qa, all 8 k-steps: lane half h holds dims 64ks + 16h +
      // [0,16) and 64ks + 32 + 16h + [0,16); byte j of qs[term][k] scales k-step 4k + j
      i32x8 qf[2][8];
      uint32_t qs[2][2];
      {
        const int head = 32 * qa + lrow, sw = head & 15;
#pragma unroll
        for (int term = 0; term < 2; ++term) {
          const unsigned char* row = smem + C::OFF_QT + (term * HP + head) * 512;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * ((4 * ks + lhalf) ^ sw));
            const uint4 hi = *reinterpret_cast<const uint4*>(row + 16 * ((4 * ks + 2 + lhalf) ^ sw));
            qf[term][ks] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
          const unsigned char* qsr = smem + C::OFF_QSC + (term * HP + head) * 16;
          qs[term][0] = scale_word<C>(qsr, 0, hsel);
          qs[term][1] = scale_word<C>(qsr, 1, hsel);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // the first tile landed
      __syncthreads();  // B_B: q tile read (the P.V waves overwrite it), first tile visible

      const int n = I.n;
      // The running max starts as a reference of 8 (scores are in log2 units; P stays at
      // most 1 below it and at most 2^8 below the raise threshold m + 8): exp2(s - m) is
      // exact for any reference both row halves share, so a tile needs the merge of the
      // halves' maxima (the slow path) only when a block max exceeds m + 8, or, while no
      // valid row has been seen yet (mref), lies below m - 64 (the reference is then
      // replaced by the merged max; nothing has been accumulated, so the rescale is 0).
      // mref is cleared from the merged block maxima, which both halves read, so the
      // halves always agree on it.
      float m_run = 8.f, l_run = 0.f, l_pend = 0.f;
      bool mref = true;
      f32x16 s;  // scores of the last tile, kept for a rewrite of its P
      // flag check for tile it - 1 (it >= 1): the slow path merges the block maxima,
      // raises the running max and rewrites P
      auto check = [&](const int it) __attribute__((always_inline)) {
        const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
        const int head = 32 * qa + lrow;
        {
          const int4 fl = *reinterpret_cast<const int4*>(flag_l + 4 * ((it - 1) & 1));
          if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
            // slow path for tile it - 1: merge the block maxima, raise the running max
            const float* mx = maxx + 2 * HP * ((it - 1) & 1);
            const float mt = fmaxf(mx[head], mx[HP + head]);
            float mnew = m_run;
            if (mt > -INFINITY && (mref || mt > m_run + 8.0f)) mnew = mt;
            const float alpha = mref ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
            if (mt > -INFINITY) mref = false;
            const bool raised = __any(mnew != m_run);
            m_run = mnew;
            const float msafe = mnew;
            float p[16];
            float lp = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              p[i] = __builtin_amdgcn_exp2f(s[i] - msafe);
              lp += p[i];
            }
            l_run = l_run * alpha + lp;
            unsigned char* prow = p_buf(it - 1) + head * 128;
            const int sw = swz(head);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              *reinterpret_cast<uint4*>(prow + 16 * ((4 * qc + 2 * kk + lhalf) ^ sw)) =
                  make_uint4(pack_bf16(p[8 * kk], p[8 * kk + 1]), pack_bf16(p[8 * kk + 2], p[8 * kk + 3]),
                             pack_bf16(p[8 * kk + 4], p[8 * kk + 5]), pack_bf16(p[8 * kk + 6], p[8 * kk + 7]));
            if (qc == 0 && lhalf == 0) alpha_l[head] = alpha;
            if (qc == 0 && lane == 0) flag_l[8 + qa] = raised ? 1 : 0;
            __syncthreads();  // B': P and alpha rewritten
          } else {
            l_run += l_pend;
            if (mref) {
              const float* mx = maxx + 2 * HP * ((it - 1) & 1);
              if (fmaxf(mx[head], mx[HP + head]) > -INFINITY) mref = false;
            }
          }
        }
      };
      // tile after which the next item's q is touched (none without a next item)
      const int touch_it = next < total ? (n >= 2 ? n - 2 : 0) : -1;
      uint32_t tch0 = 0, tch1 = 0;
      for (int it = 0; it < n; ++it) {
        const int tile = I.tb + it;
        const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
        const int head = 32 * qa + lrow;
        const int r = 32 * qc + lrow;
        i32x8 A[8];
        uint32_t ksc0 = 0, ksc1 = 0;
        auto load_a = [&](int ks0) {
          const unsigned char* raw_l = raw_buf(it);
#pragma unroll
          for (int ks = ks0; ks < ks0 + 4; ++ks) {
            const uint4 lo = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(r, 4 * ks + lhalf));
            const uint4 hi = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(r, 4 * ks + 2 + lhalf));
            A[ks] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
        };
        if (it > 0) check(it);
        const int id_cur = valid_id(I, tile, raw_cur);
        const unsigned long long mask = __ballot(id_cur >= 0);
        const int raw_next2 = fetch_id(I, tile + 2);
#ifdef SMLA_DEBUG_CHECKS
        if (w == 0)
          debug_flag_tile(a.sched, a.n_rows, tile < I.te && tile * T + lane < I.lcap, raw_cur, id_cur >= 0,
                          sc_buf(it) + C::NSB * lane, C::NSB);
#endif
        // (the next tile's DMA is issued by the P.V waves, whose loop has more slack)
        // the next item's q rows into the L2, two tiles ahead of its prologue (one 128-byte
        // line per load, 64 KB per workgroup; heads >= h_q read nothing).  Issued after
        // this tile's DMA, so the end of this iteration waits for the DMA only.
        const bool touch = it == touch_it;
        if (touch) {
          const __amdgpu_buffer_rsrc_t qrs =
              buf_rsrc(a.q + (size_t)((a.order ? a.order[next] : next) / ns) * a.h_q * D, (uint32_t)(a.h_q * D * 2));
          const uint32_t off = 256u * (uint32_t)(64 * w + lane);
          tch0 = __builtin_amdgcn_raw_buffer_load_b32(qrs, off, 0, 0);
          tch1 = __builtin_amdgcn_raw_buffer_load_b32(qrs, off + 128u, 0, 0);
        }
        {
          const unsigned char* sc_l = sc_buf(it);
          const uint32_t hsel = lhalf ? 0x07050301u : 0x06040200u;
          ksc0 = scale_word<C>(sc_l + r * C::NSB, 0, hsel);
          ksc1 = scale_word<C>(sc_l + r * C::NSB, 1, hsel);
          load_a(0);
          load_a(4);
          qk_block<4, true>(s, A, qf[0], qf[1], ksc0, qs[0][0], qs[1][0]);
          qk_block<4, false>(s, A + 4, qf[0] + 4, qf[1] + 4, ksc1, qs[0][1], qs[1][1]);
        }
        {
          qk_drain(s);
          // mask (row 32qc + 8g + 4h + j holds value 4g + j), block max over the 32 rows
          const uint32_t mw = (uint32_t)(mask >> (32 * qc));
          float lm = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rr = 8 * (i >> 2) + (i & 3);
            const unsigned long long lmk = (((mw >> rr) & 1u) ? 0x00000000FFFFFFFFull : 0ull) |
                                           (((mw >> (rr + 4)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
            s[i] = __builtin_amdgcn_inverse_ballot_w64(lmk) ? s[i] : -INFINITY;
            lm = fmaxf(lm, s[i]);
          }
          lm = pair_max(lm);
          // P against the running max; exact unless the flag below sends the tile to the
          // slow path, which rewrites it
          const float msafe = m_run;
          float p[16];
          float lp = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(s[i] - msafe);
            lp += p[i];
          }
          l_pend = lp;
          unsigned char* prow = p_buf(it) + head * 128;
          const int sw = swz(head);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            *reinterpret_cast<uint4*>(prow + 16 * ((4 * qc + 2 * kk + lhalf) ^ sw)) =
                make_uint4(pack_bf16(p[8 * kk], p[8 * kk + 1]), pack_bf16(p[8 * kk + 2], p[8 * kk + 3]),
                           pack_bf16(p[8 * kk + 4], p[8 * kk + 5]), pack_bf16(p[8 * kk + 6], p[8 * kk + 7]));
          if (lhalf == 0) maxx[2 * HP * (it & 1) + qc * HP + head] = lm;
          const bool over = __any(lm > m_run + 8.0f || (mref && lm > -INFINITY && lm < m_run - 64.0f));
          if (lane == 0) flag_l[4 * (it & 1) + w] = over ? 1 : 0;
        }
        // this wave's index loads landed (vmcnt(0); vmcnt(2) behind the q touches)
        if (touch)
          __builtin_amdgcn_s_waitcnt(0x0F72);
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);
        raw_cur = raw_next;
        raw_next = raw_next2;
        __syncthreads();  // end of iteration
      }
      // last iteration (P.V of the last tile on the other waves): final check, the item's
      // row sums and max for the epilogue, and the next item's ids, which stay in flight
      // into the next item's prologue
      uint4 x[4][4];
      {
        if (n > 0) check(n);
        const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
        const int head = 32 * qa + lrow;
        const float lw = pair_sum(l_run);
        if (lhalf == 0) lsum[qc * HP + head] = lw;
        if (qc == 0 && lhalf == 0) mfin[head] = m_run;
        if (next < total) {
          I = info(next);
          raw_cur = fetch_id(I, I.tb);
          raw_next = fetch_id(I, I.tb + 1);
        }
        __syncthreads();  // end of the last iteration
      }
      item = next;
      if (item >= total) break;
      // the first ids are resolved before the q loads go out, so that the compiler's wait
      // for them does not wait for q as well
      const int id0 = valid_id(I, I.tb, raw_cur);
      q_load(I, std::integral_constant<int, 4>{}, x);
      transition(std::integral_constant<int, 4>{}, x, id0);
      asm volatile("" ::"v"(tch0), "v"(tch1));  // the touches' results are never looked at
    }
    // this workgroup is done; the last one to finish leaves the counters zero for the
    // next call on this workspace
    if (w == 0 && (((int)threadIdx.x + opaque_zero()) & 63) == 0) {
      if (atomicAdd(a.sched + 1, 1u) == gridDim.x - 1) {
        atomicExch(a.sched, 0u);
        atomicExch(a.sched + 1, 0u);
      }
    }
  } else {
    // =============================== P.V waves
    const int v = w - 4;
    int item = blockIdx.x;
    Item I = info(item);
    {
      // the first item's prologue is shared with the QK waves (heads 16..31, 48..63);
      // this wave's table also serves the epilogue's inverse RoPE
      uint4 x[4][4];
      q_load(I, std::integral_constant<int, 2>{}, x);
      setup();
      rope_tab(I);
      q_units(std::integral_constant<int, 2>{}, x);
    }
    while (true) {
      __syncthreads();  // B_A
      const int next = __builtin_amdgcn_readfirstlane(flag_l[12]);
      __syncthreads();  // B_B
      const int n = I.n;
      // O^T of this wave's 128 dims: acc[mb][nb] is dims 32 nb .. 32 nb + 31 x heads
      // 32 mb .. 32 mb + 31 (Vt as the A operand, P as B), so lane = head 32 mb + lrow and
      // register i = dim 32 nb + 8 (i >> 2) + 4 lhalf + (i & 3): each 32-dim output block
      // of a head lives in one lane pair (lane, lane ^ 32)
      f32x16 acc[2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
      int raw_next = fetch_id(I, I.tb + 1);

      // One iteration: P.V of tile it - 1 (PV) and / or this wave's DMA parts of tile it + 1
      // (DM).  V is never written back to LDS: the scaled E4M3 MFMA of the raw rows (A,
      // with their UE8M0 block scales) against an identity (B, E4M3 1.0, scale 1) gives the
      // dequantized block exactly in f32, in the MFMA output layout lane = dim, register i
      // = slot 8 (i >> 2) + 4 lhalf + (i & 3) of a 32-slot half.  The P.V contraction takes
      // the slots in that order: k-step ks, lane half kg holds slots 16 ks + 4 kg + {0..3}
      // and 16 ks + 8 + 4 kg + {0..3} (registers 0..7 of the half's output for the even
      // k-step, 8..15 for the odd one, rounded to bf16, which is exact), and the QK waves
      // store P in the same order.  So the transposition costs one MFMA per 32 x 32 block and
      // a bf16 pack per value pair, and no LDS traffic beyond reading the raw rows once.
      auto pv_iter = [&](const int it, auto pv_c, auto dm_c) __attribute__((always_inline)) {
        constexpr bool PV = decltype(pv_c)::value, DM = decltype(dm_c)::value;
        const int tile = I.tb + it;
        const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
        const unsigned char* p_l = p_buf(it - 1);
        const unsigned char* raw_l = raw_buf(it - 1);
        const unsigned char* sc_l = sc_buf(it - 1);
        // P rows (heads) are 128 bytes, 16-byte chunk ch stored at ch ^ swz(head); for head
        // 32 mb + lrow and ch = 2 ks + lhalf that is nu ^ 2ks ^ 4mb (nu = swz(lrow) ^ lhalf)
        const int nu = (lrow & 7) ^ (lrow >> 3) ^ lhalf;
        uint32_t rd[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) rd[c] = 128 * lrow + 16 * (nu ^ c);
        const int raw_next2 = fetch_id(I, tile + 2);
        const int id_next = valid_id(I, tile + 1, raw_next);
        bf16x8 Ap[2][2];  // P of k-steps 2 sh + kk, head blocks mb
        auto load_p = [&](int sh) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              Ap[kk][mb] = *reinterpret_cast<const bf16x8*>(p_l + 4096 * mb + rd[(2 * (2 * sh + kk)) ^ (4 * mb)]);
        };
        if constexpr (PV) {
          load_p(0);
          const int4 fl = *reinterpret_cast<const int4*>(flag_l + 4 * ((it - 1) & 1));
          if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
            __syncthreads();  // B': P and alpha rewritten
            load_p(0);
            const int2 rf = *reinterpret_cast<const int2*>(flag_l + 8);
            if (__builtin_amdgcn_readfirstlane(rf.x | rf.y)) {
#pragma unroll
              for (int mb = 0; mb < 2; ++mb) {
                const float al = alpha_l[32 * mb + lrow];  // one head per lane
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                  for (int i = 0; i < 16; ++i) acc[mb][nb][i] *= al;
              }
            }
          }
          // identity operands: lane (column n = lrow, half h) holds K = 16 h + p (p < 16)
          // and K = 32 + 16 h + (p - 16) (p >= 16); E4M3 1.0 where K = n (block 0 of the
          // 64-dim step) or K = 32 + n (block 1)
          int i4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = lrow - 16 * lhalf - 4 * q;
            i4[q] = (idx >= 0 && idx < 4) ? (0x38 << (8 * idx)) : 0;
          }
          const i32x8 ilo = {i4[0], i4[1], i4[2], i4[3], 0, 0, 0, 0};
          const i32x8 ihi = {0, 0, 0, 0, i4[0], i4[1], i4[2], i4[3]};
          const int unit = 0x7F7F7F7F;
          __builtin_amdgcn_s_setprio(2);
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            if (sh == 1) load_p(1);
            // raw rows 32 sh + lrow; their scales of blocks 4v .. 4v + 3, byte j of the word
            // for lane half h = block 4v + 2j + h (the A scale of k-block h of chunk j)
            const int r = 32 * sh + lrow;
            const uint32_t w4 = *reinterpret_cast<const uint32_t*>(sc_l + r * C::NSB + 4 * v);
            const uint32_t asc = __builtin_amdgcn_perm(w4, w4, lhalf ? 0x07050301u : 0x06040200u);
            static_for<2>([&](auto kc_c) {
              constexpr int kc = decltype(kc_c)::value;
              // this wave's share of the next tile's DMA and that of its SIMD's QK wave
              // (w - 4): rows 32 (w - 4) + 8 (2 sh + kc) .. + 7 and 128 + ..., scales last
              if constexpr (DM) {
                dma_part(2 * sh + kc, w, id_next, raw_buf(it + 1), sc_buf(it + 1), std::false_type{});
                dma_part(2 * sh + kc, w - 4, id_next, raw_buf(it + 1), sc_buf(it + 1), std::false_type{});
                if (sh == 1 && kc == 1) dma_part(4, w - 4, id_next, raw_buf(it + 1), sc_buf(it + 1), std::false_type{});
              }
              const int ks8 = 2 * v + kc;  // 64-dim step of the row
              const uint4 lo = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(r, 4 * ks8 + lhalf));
              const uint4 hi = *reinterpret_cast<const uint4*>(raw_l + raw_off<C>(r, 4 * ks8 + 2 + lhalf));
              const i32x8 A = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
              const f32x16 zero = {};
              f32x16 tv[2];
              tv[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, ilo, zero, 0, 0, kc, (int)asc, 0, unit);
              tv[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, ihi, zero, 0, 0, kc, (int)asc, 0, unit);
#pragma unroll
              for (int t = 0; t < 2; ++t) {
                const int nb = 2 * kc + t;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                  const f32x16& x = tv[t];
                  // bf16 of exactly representable values (4 significant bits): the RNE pack
                  // is exact.  (A v_perm of the f32 high halves would be as exact, but the
                  // compiler folds a perm of two elements of an MFMA result into one.)
                  const uint32_t b0 = pack_bf16(x[8 * kk], x[8 * kk + 1]);
                  const uint32_t b1 = pack_bf16(x[8 * kk + 2], x[8 * kk + 3]);
                  const uint32_t b2 = pack_bf16(x[8 * kk + 4], x[8 * kk + 5]);
                  const uint32_t b3 = pack_bf16(x[8 * kk + 6], x[8 * kk + 7]);
                  const bf16x8 bv = __builtin_bit_cast(bf16x8, make_uint4(b0, b1, b2, b3));
#pragma unroll
                  for (int mb = 0; mb < 2; ++mb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, Ap[kk][mb], acc[mb][nb], 0, 0, 0);
                }
              }
            });
          }
          __builtin_amdgcn_s_setprio(0);
        } else if constexpr (DM) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            dma_part(k, w, id_next, raw_buf(it + 1), sc_buf(it + 1), std::false_type{});
            dma_part(k, w - 4, id_next, raw_buf(it + 1), sc_buf(it + 1), std::false_type{});
          }
          dma_part(4, w - 4, id_next, raw_buf(it + 1), sc_buf(it + 1), std::false_type{});
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        raw_next = raw_next2;
        __syncthreads();  // end of iteration
      };
      // the first and last iterations are separate straight-line copies
      if (n == 0) {
        pv_iter(0, std::false_type{}, std::false_type{});
      } else {
        pv_iter(0, std::false_type{}, std::true_type{});
        for (int it = 1; it < n; ++it) pv_iter(it, std::true_type{}, std::true_type{});
        pv_iter(n, std::true_type{}, std::false_type{});
      }

      // ---- finish of the item
      const bool more = next < total;
      Item In = I;
      if (more) In = info(next);
      const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
      const auto& K = karg();
      const int hq = K.h_q;
      if (ns == 1) {
        // Straight from the registers: per head (lane) and 32-dim block (nb) the lane pair
        // (lane, lane ^ 32) holds the block, 16 dims each.  Normalize by the head's row sum,
        // inverse RoPE (blocks 14 and 15 sit in nb 2 and 3 of the last wave: the pair
        // (448 + j, 480 + j) is the same register of the same lane), block amax over the
        // pair, UE8M0 exponent, E4M3 codes; the pair then swaps two code words so that
        // each lane stores 16 consecutive bytes (lhalf 0: dims 0..15 of the block, lhalf
        // 1: dims 16..31).
        uint8_t* out_fp8 = K.out_fp8;
        uint8_t* out_scales = K.out_scales;
        float* out_f32 = K.out_f32;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int h = 32 * mb + lrow;
          const float lt = lsum[h] + lsum[HP + h];
          const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][nb][i] *= inv;
          if (rot && v == 3) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 c4 = *reinterpret_cast<const float4*>(rtab + 8 * g + 4 * lhalf);
              const float4 s4 = *reinterpret_cast<const float4*>(rtab + 32 + 8 * g + 4 * lhalf);
              const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                const float x0 = acc[mb][2][4 * g + jj], x1 = acc[mb][3][4 * g + jj];
                acc[mb][2][4 * g + jj] = __builtin_fmaf(x1, sv[jj], x0 * cc[jj]);
                acc[mb][3][4 * g + jj] = __builtin_fmaf(-x0, sv[jj], x1 * cc[jj]);
              }
            }
          }
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int gb = 4 * v + nb;
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[mb][nb][i]));
            amax = pair_max(amax);
            const int e8 = ue8m0_exp(amax);
            const float sc = ue8m0_f32((uint32_t)e8);  // codes = RNE(o / 2^(e-127))
            uint32_t wd[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
              wd[g] = enc2(enc2(0u, acc[mb][nb][4 * g], acc[mb][nb][4 * g + 1], sc, false), acc[mb][nb][4 * g + 2],
                           acc[mb][nb][4 * g + 3], sc, true);
            // word g holds dims 8g + 4 lhalf .. + 3: lhalf 0 keeps g = 0, 1 and takes the
            // partner's, lhalf 1 keeps g = 2, 3
            const uint32_t give0 = lhalf ? wd[0] : wd[2], give1 = lhalf ? wd[1] : wd[3];
            const uint32_t got0 = xor32_u32(give0), got1 = xor32_u32(give1);
            const uint4 st = lhalf ? make_uint4(got0, wd[2], got1, wd[3]) : make_uint4(wd[0], got0, wd[1], got1);
            if (h < hq) {
              const size_t g0 = ((size_t)I.t * hq + h) * D + 32 * gb;
              *reinterpret_cast<uint4*>(out_fp8 + g0 + 16 * lhalf) = st;
              if (lhalf == 0) out_scales[((size_t)I.t * hq + h) * (D / 32) + gb] = (uint8_t)e8;
              if (out_f32) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                  *reinterpret_cast<float4*>(out_f32 + g0 + 8 * g + 4 * lhalf) =
                      make_float4(acc[mb][nb][4 * g], acc[mb][nb][4 * g + 1], acc[mb][nb][4 * g + 2],
                                  acc[mb][nb][4 * g + 3]);
              }
            }
          }
        }
      } else {
        // this split's (acc, m, l) for the combine kernel, the accumulator in register
        // order: each store instruction writes 1 KB contiguously
        const int split = item % ns;
        float* part = K.ws + ((size_t)I.t * ns + split) * partial_floats_d(hq, D);
        float* pm = part + WSP_M;
        float* pl = part + WSP_L;
        if (v == 0 && lane < hq) {
          // a split that read nothing (l = 0) reports m = -inf: the combine skips it and
          // never reads its accumulator
          const float lt = lsum[lane] + lsum[HP + lane];
          pm[lane] = lt > 0.f ? mfin[lane] : -INFINITY;
          pl[lane] = lt;
        }
        // the token's cos / sin table (this wave's, the one its epilogue would use)
        if (rot && v == 3 && lane < 32) {
          part[WSP_ROPE + lane] = rtab[lane];
          part[WSP_ROPE + 32 + lane] = rtab[32 + lane];
        }
        if (n > 0) {
          uint4* pv4 = reinterpret_cast<uint4*>(part) + 2 * 4 * 2 * 64 * v + lane;
          float* psc = part + WSP_SCL;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              float am = 0.f;
#pragma unroll
              for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(acc[mb][nb][i]));
              am = pair_max(am);
              float enc, dec;
              f16_block_scale(am, enc, dec);
              if (lane < 32) psc[(4 * v + nb) * HP + 32 * mb + lrow] = dec;
#pragma unroll
              for (int g2 = 0; g2 < 2; ++g2) {
                const int r = 8 * g2;
                pv4[((mb * 4 + nb) * 2 + g2) * 64] = make_uint4(
                    pack_f16(acc[mb][nb][r] * enc, acc[mb][nb][r + 1] * enc),
                    pack_f16(acc[mb][nb][r + 2] * enc, acc[mb][nb][r + 3] * enc),
                    pack_f16(acc[mb][nb][r + 4] * enc, acc[mb][nb][r + 5] * enc),
                    pack_f16(acc[mb][nb][r + 6] * enc, acc[mb][nb][r + 7] * enc));
              }
            }
        }
      }
      if (!more) break;
      item = next;
      I = In;
      rope_tab(I);
    }
  }
}

// ---------------------------------------------------------------------------------------
// The step over the two-pool nvfp4_ds_mla cache, d = 512: entries j < swa_entries of an
// index row name rows of the E4M3 + UE8M0 SWA pool (512 codes + 16 scales), the later
// entries rows of the NVFP4 pool (256 bytes of E2M1 pairs + 32 E4M3 scales, one per 16
// elements) [vLLM #56344 "Deepseek V41 Attention MegaKernel", Purpose: fp8 528 B SWA rows
// + fp4 288 B compressed rows].  An E2M1 value times an E4M3 scale has up to six
// significant bits and its scale is not a power of two, so neither the scaled FP8 MFMA nor
// an E4M3 re-encoding holds it exactly; both kinds of rows are decoded exactly to bf16
// instead, and q' is bf16, with QK^T and P.V on bf16 MFMAs.
//
// One 512-thread workgroup per (token, split).  Per 64-entry tile (each tile lies in one
// segment: swa_entries is a multiple of 64):
//   gather    thread (row gr = tid / 8, part gp = tid % 8) loads dims 64 gp .. 64 gp + 63 of
//             its row (64 E4M3 bytes + 2 UE8M0 scales, or 32 bytes of E2M1 pairs + 4 E4M3
//             scales) through range-checked buffer loads (rows that are not read come in as
//             zeros), one tile ahead, and writes them as bf16 into the V tile [slot][dim]
//             (16-byte chunk c of a slot's row stored at chunk c ^ ((c >> 3) & 7), so that
//             the eight threads of a row write distinct banks);
//   QK^T      wave (qa, qc, qd) computes the partial S^T[32 slots of half qc][32 heads of
//             group qa] over dim half qd (16 bf16 MFMAs, q' fragments in VGPRs); the qd = 1
//             halves meet the qd = 0 halves through LDS;
//   softmax   the qd = 0 waves mask, take the tile max of each head over both slot halves
//             (LDS), raise the running max, write P = exp2(s - m) in bf16 and the rescale;
//   P.V       wave w owns output dims [64 w, 64 w + 64) of all 64 heads: O^T += V^T P^T with
//             the V^T operand read by the 16-bit transpose load (ds_read_b64_tr_b16: lane
//             i of a 16-lane group receives element i % 4 of the 8-byte pieces addressed by
//             lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12, which turns four row-major slots
//             of 16 dims into 16 lanes of four slots each).
// Then the same epilogue as the generic kernel, or the split partials: at rotary widths 0
// and 64 in smla_ws's f16 register-order format for smla_combine_lm4 / lm1, else in the
// generic f32 format for smla_combine.
struct NvCfg {
  static constexpr int kD = 512, kEB = 2;  // the q prologue writes a bf16 q' tile
  static constexpr int D = kD;
  static constexpr int QS = D + 8;         // bf16 stride of the q' tile and of the V tile
  static constexpr int VS = QS;
  static constexpr int OFF_Q = 0, OFF_V = 0;
  static constexpr int V_BYTES = T * VS * 2;
  static constexpr int OFF_SX = V_BYTES;                 // partial S^T of the qd = 1 waves
  static constexpr int PS = T + 8;                       // bf16 stride of the P tile
  static constexpr int OFF_P = OFF_SX + 4 * 64 * 16 * 4;
  static constexpr int LOOP_END = OFF_P + HP * PS * 2;
  static constexpr int OS = D + 4;                       // f32 stride of the epilogue's o tile
  static constexpr int O_BYTES = HP * OS * 4;
  static constexpr int OFF_SMALL = align16(cmax(O_BYTES, LOOP_END));
  static constexpr int OFF_COS = OFF_SMALL;
  static constexpr int OFF_SIN = OFF_COS + (D / 2) * 4;
  static constexpr int OFF_MAXX = OFF_SIN + (D / 2) * 4;  // [2 slot halves][HP]
  static constexpr int OFF_ALPHA = OFF_MAXX + 2 * HP * 4;     // [HP]
  static constexpr int OFF_LSUM = OFF_ALPHA + HP * 4;         // [2 slot halves][HP]
  static constexpr int OFF_VALID = OFF_LSUM + 2 * HP * 4;     // [T]: the tile's entry is read
  static constexpr int SMEM = OFF_VALID + T * 4;
  static constexpr int MAX_ROPE = (LOOP_END - OFF_SX) / (HP * 4) - 4;  // the prologue's staging over SX + P
  static_assert(HP * QS * 2 <= OFF_SX && SMEM <= 160 * 1024, "LDS layout");
  static_assert(MAX_ROPE >= 64, "rotary staging");
};

__global__ __launch_bounds__(NTHREADS, 1) void smla_nv(KArgs a) {
  using C = NvCfg;
  constexpr int D = C::D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];
  float* cs = reinterpret_cast<float*>(smem + C::OFF_COS);
  float* sn = reinterpret_cast<float*>(smem + C::OFF_SIN);
  float* maxx = reinterpret_cast<float*>(smem + C::OFF_MAXX);
  float* alpha_l = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
  float* lsum = reinterpret_cast<float*>(smem + C::OFF_LSUM);
  int* valid_l = reinterpret_cast<int*>(smem + C::OFF_VALID);
  unsigned char* vt = smem + C::OFF_V;
  unsigned char* pt = smem + C::OFF_P;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int qa = w & 1, qc = (w >> 1) & 1, qd = w >> 2;  // QK roles
  const int ns = a.num_splits;
  // the item of this workgroup: in the order smla_order wrote (tokens by descending tile
  // count, so that the dispatcher, which starts workgroups in id order as compute units
  // free up, takes the long ones first), or item = id
  const int item = a.order ? a.order[blockIdx.x] : (int)blockIdx.x;
  const int t = item / ns, split = item % ns;
  const int pos = a.positions[t];
  const int lraw = a.topk_length[t];
  const int lcap = lraw < 0 ? 0 : (lraw > a.topk ? a.topk : lraw);
  const int ntile = (lcap + T - 1) / T;
  const int tb = split * a.tiles_per_split;
  const int te_raw = tb + a.tiles_per_split;
  const int te = te_raw < ntile ? te_raw : ntile;

  // gather role: row gr of the tile, dims 64 gp .. 64 gp + 63
  const int gr = tid >> 3, gp = tid & 7;
  const __amdgpu_buffer_rsrc_t idx_rs = buf_rsrc(a.indices + (size_t)t * a.topk, (uint32_t)a.topk * 4u);
  const __amdgpu_buffer_rsrc_t swa_rs = buf_rsrc(a.pool, (uint32_t)(a.n_rows * D));
  const __amdgpu_buffer_rsrc_t swa_srs = buf_rsrc(a.scales, (uint32_t)(a.n_rows * (D / 32)));
  const __amdgpu_buffer_rsrc_t cmp_rs = buf_rsrc(a.cmp_pool, (uint32_t)(a.n_cmp * (D / 2)));
  const __amdgpu_buffer_rsrc_t cmp_srs = buf_rsrc(a.cmp_scales, (uint32_t)(a.n_cmp * (D / 16)));
  // the raw id of entry tile * 64 + gr (an entry past the row reads 0; decided in row_of)
  auto fetch_id = [&](int tile) -> int {
    const int j = tile * T + gr;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(idx_rs, (uint32_t)(j < a.topk ? j : a.topk) * 4u, 0, 0);
  };
  // the row entry tile * 64 + gr reads, or -1 (past the length, a sentinel, out of its pool)
  auto row_of = [&](int tile, int raw) -> int {
    const int j = tile * T + gr;
    const long long n = j < a.swa_entries ? a.n_rows : a.n_cmp;
    return (tile < te && j < lcap && raw >= 0 && (long long)raw < n) ? raw : -1;
  };
  struct Raw {
    uint4 c[4];
    uint32_t s;
  };
  auto gather = [&](int tile, int id, Raw& g) {
    if (tile * T < a.swa_entries) {
      // every chunk's offset is selected on its own: kNoRow plus a chunk offset would wrap
      // round to the start of the pool
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t off = id >= 0 ? (uint32_t)id * D + 64u * gp + 16u * k : kNoRow;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(swa_rs, off, 0, 0);
        g.c[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      g.s = __builtin_amdgcn_raw_buffer_load_b16(swa_srs, id >= 0 ? (uint32_t)id * (D / 32) + 2u * gp : kNoRow, 0, 0);
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t off = id >= 0 ? (uint32_t)id * (D / 2) + 32u * gp + 16u * k : kNoRow;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(cmp_rs, off, 0, 0);
        g.c[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      g.c[2] = g.c[3] = make_uint4(0u, 0u, 0u, 0u);
      g.s = __builtin_amdgcn_raw_buffer_load_b32(cmp_srs, id >= 0 ? (uint32_t)id * (D / 16) + 4u * gp : kNoRow, 0, 0);
    }
  };
  // the gathered part of row gr as bf16 into the V tile (exact: an E4M3 value times a
  // power of two in the range the ABI admits, or an E2M1 value times an E4M3 scale)
  auto dequant = [&](int tile, const Raw& g) {
    // 16-byte chunk i of this thread's part (chunk 8 gp + i of the row) at i ^ gp: the
    // eight threads of a row then write eight different bank groups at each step
    uint4* dst = reinterpret_cast<uint4*>(vt + (gr * C::VS + 64 * gp) * 2);
    auto at = [&](int i) -> uint4& { return dst[i ^ gp]; };
    if (tile * T < a.swa_entries) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float sc = ue8m0_f32((g.s >> (k < 2 ? 0 : 8)) & 0xFFu);
        const uint32_t u[4] = {g.c[k].x, g.c[k].y, g.c[k].z, g.c[k].w};
        at(2 * k) = make_uint4(cvt_lo(u[0], sc), cvt_hi(u[0], sc), cvt_lo(u[1], sc), cvt_hi(u[1], sc));
        at(2 * k + 1) = make_uint4(cvt_lo(u[2], sc), cvt_hi(u[2], sc), cvt_lo(u[3], sc), cvt_hi(u[3], sc));
      }
    } else {
      // the four E4M3 block scales, decoded exactly
      const f32x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(g.s, 1.0f, false);
      const f32x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(g.s, 1.0f, true);
      const float scv[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t u[4] = {g.c[k].x, g.c[k].y, g.c[k].z, g.c[k].w};
        // bytes 16k .. 16k + 15: elements 32k .. 32k + 31, blocks 2k, 2k + 1
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sc = scv[2 * k + (q >> 1)];
          uint32_t pk[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            // byte b of word q: elements 2b (low nibble) and 2b + 1 (high nibble), exact at
            // scale 1; the block scale is a plain f32 product (exact: 2 x 4 significant bits)
            f32x2 e2;
            if (b == 0) e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u[q], 1.0f, 0);
            else if (b == 1) e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u[q], 1.0f, 1);
            else if (b == 2) e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u[q], 1.0f, 2);
            else e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u[q], 1.0f, 3);
            pk[b] = pack_bf16(e2[0] * sc, e2[1] * sc);
          }
          at(4 * k + q) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      }
    }
  };

  // ---------------- prologue: q' (bf16, times sm_scale log2 e) into the q tile
  int raw_cur = tb < te ? fetch_id(tb) : -1;
  Raw g;
  float* ystage = reinterpret_cast<float*>(smem + C::OFF_SX);
  q_prologue<C>(smem, t, pos, a, cs, sn, ystage, [&]() {});
  __syncthreads();
  // q' fragments (B operand of S^T = K q'^T): head 32 qa + lrow, k-steps 16 qd .. 16 qd + 15,
  // lane half h holding dims 16 ks + 8 h .. + 7
  bf16x8 qf[16];
  {
    const unsigned short* qrow = reinterpret_cast<const unsigned short*>(smem + C::OFF_Q) + (32 * qa + lrow) * C::QS;
#pragma unroll
    for (int j = 0; j < 16; ++j) qf[j] = *reinterpret_cast<const bf16x8*>(qrow + 16 * (16 * qd + j) + 8 * lhalf);
  }
  // the first tile's rows (after the q tile is read: the V tile shares its space)
  if (tb < te) gather(tb, row_of(tb, raw_cur), g);
  int raw_next = tb + 1 < te ? fetch_id(tb + 1) : -1;
  __syncthreads();  // q fragments loaded: the V tile may overwrite the q tile

  // P.V accumulators of this wave's 64 dims: acc[mb][nb] = O^T rows (dims 64 w + 32 nb ..)
  // x columns (heads 32 mb ..): lane = head, register i = dim 8 (i >> 2) + 4 lhalf + (i & 3)
  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // qd = 0 waves: per head (lane), this slot half

  for (int tile = tb; tile < te; ++tile) {
    const int lane = ((int)threadIdx.x + opaque_zero()) & 63, lrow = lane & 31, lhalf = lane >> 5;
    dequant(tile, g);
    if (gp == 0) valid_l[gr] = row_of(tile, raw_cur) >= 0;
    __syncthreads();  // V tile and the read mask complete
    // next tile's rows, landing during this tile's arithmetic
    if (tile + 1 < te) gather(tile + 1, row_of(tile + 1, raw_next), g);
    const int raw_next2 = tile + 2 < te ? fetch_id(tile + 2) : -1;

    // ---- QK^T: partial S^T[32 slots of half qc][32 heads of group qa] over dim half qd
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    {
      const unsigned short* krow = reinterpret_cast<const unsigned short*>(vt) + (32 * qc + lrow) * C::VS;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // chunk c = 2 (16 qd + j) + lhalf of the row, stored at c ^ ((c >> 3) & 7)
        const int c = 2 * (16 * qd + j) + lhalf;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 8 * (c ^ ((c >> 3) & 7)));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[j], s, 0, 0, 0);
      }
    }
    float* sx = reinterpret_cast<float*>(smem + C::OFF_SX) + (2 * qa + qc) * 1024;
    if (qd == 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sx[i * 64 + lane] = s[i];
    }
    __syncthreads();  // partial S^T of the qd = 1 waves visible
    if (qd == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] += sx[i * 64 + lane];
      // slot 32 qc + 8 (i >> 2) + 4 lhalf + (i & 3) counts only if its entry is read
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = 32 * qc + 8 * (i >> 2) + 4 * lhalf + (i & 3);
        s[i] = valid_l[slot] ? s[i] : -INFINITY;
        lm = fmaxf(lm, s[i]);
      }
      lm = pair_max(lm);
      if (lhalf == 0) maxx[qc * HP + 32 * qa + lrow] = lm;
    }
    __syncthreads();  // block maxima of both slot halves visible
    if (qd == 0) {
      const int head = 32 * qa + lrow;
      const float mt = fmaxf(maxx[head], maxx[HP + head]);
      const float mnew = fmaxf(m_run, mt);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      float p[16], lp = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - msafe);
        lp += p[i];
      }
      l_run = l_run * alpha + lp;
      m_run = mnew;
      // P [head][slot] in bf16, natural slot order
      unsigned short* prow = reinterpret_cast<unsigned short*>(pt) + head * C::PS + 32 * qc + 4 * lhalf;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2*>(prow + 8 * g4) =
            make_uint2(pack_bf16(p[4 * g4], p[4 * g4 + 1]), pack_bf16(p[4 * g4 + 2], p[4 * g4 + 3]));
      if (qc == 0 && lhalf == 0) alpha_l[head] = alpha;
    }
    __syncthreads();  // P and the rescale visible
    // ---- P.V: O^T[dims 64 w .. 64 w + 63][heads] += V^T P^T
    {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const float al = alpha_l[32 * mb + lrow];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[mb][nb][i] *= al;
      }
      const int grp = lane >> 4, p16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 bp[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          bp[mb] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const unsigned short*>(pt) +
                                                    (32 * mb + lrow) * C::PS + 16 * ks + 8 * lhalf);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          // V^T fragment of dims 64 w + 32 nb .. + 31, slots 16 ks + 8 lhalf .. + 7: lane p of
          // 16-lane group g points at slot k0 + p / 4, dims 16 (g & 1) + 4 (p & 3) .. + 3
          const int dim0 = 64 * w + 32 * nb + 16 * (grp & 1) + 4 * (p16 & 3);
          // (the compiler's own transpose loads: it counts their waits, so the sixteen
          // loads of a tile need not each wait for the last)
          uint2 h0, h1;
          {
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            const int slot = 16 * ks + 8 * lhalf + (p16 >> 2);
            const int c = dim0 >> 3;  // its 16-byte chunk, stored at c ^ ((c >> 3) & 7)
            lds_s16x4* ad = (lds_s16x4*)(vt + (slot * C::VS + 8 * (c ^ ((c >> 3) & 7)) + (dim0 & 7)) * 2);
            h0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(ad));
            h1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(ad + C::VS));
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, bp[mb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
    raw_cur = raw_next;
    raw_next = raw_next2;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // next tile's rows landed
    __syncthreads();  // V tile and P read: the next tile may overwrite them
  }

  // ---------------- finish: l and m per head, then normalize + epilogue, or the partials
  if (qd == 0) {
    const float lw = pair_sum(l_run);
    if (lhalf == 0) lsum[qc * HP + 32 * qa + lrow] = lw;
    if (qc == 0 && lhalf == 0) maxx[32 * qa + lrow] = m_run;
  }
  __syncthreads();
  const int d0 = 64 * w;
  if (ns == 1) {
    float* o_l = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int h = 32 * mb + lrow;
      const float lt = lsum[h] + lsum[HP + h];
      const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          o_l[h * C::OS + d0 + 32 * nb + 8 * (i >> 2) + 4 * lhalf + (i & 3)] = acc[mb][nb][i] * inv;
    }
    __syncthreads();
    epilogue<D, NTHREADS>(o_l, C::OS, a.h_q, 0, t, a, cs, sn);
  } else if (a.rope_dim == 0 || a.rope_dim == 64) {
    // smla_ws's partial format (f16 blocks in its P.V waves' register order), read by
    // smla_combine_lm4 / lm1: this wave's acc[mb][nb] (dims 64 w + 32 nb ..) is acc[mb]
    // [2 (w & 1) + nb] of P.V wave w / 2 there, with the same element order in the block
    float* part = a.ws + ((size_t)t * ns + split) * partial_floats_d(a.h_q, D);
    if (tid < a.h_q) {
      // a split that read nothing reports m = -inf: the combine never reads its accumulator
      const float lt = lsum[tid] + lsum[HP + tid];
      part[WSP_M + tid] = lt > 0.f ? maxx[tid] : -INFINITY;
      part[WSP_L + tid] = lt;
    }
    if (a.rope_dim == 64 && tid < 32) {
      part[WSP_ROPE + tid] = cs[tid];
      part[WSP_ROPE + 32 + tid] = sn[tid];
    }
    if (te > tb) {
      uint4* pv4 = reinterpret_cast<uint4*>(part) + lane;
      float* psc = part + WSP_SCL;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          float am = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(acc[mb][nb][i]));
          am = pair_max(am);
          float enc, dec;
          f16_block_scale(am, enc, dec);
          if (lane < 32) psc[(2 * w + nb) * HP + 32 * mb + lrow] = dec;
          const int slot0 = (((w >> 1) * 2 + mb) * 4 + 2 * (w & 1) + nb) * 2;
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const int r = 8 * g2;
            pv4[(slot0 + g2) * 64] = make_uint4(
                pack_f16(acc[mb][nb][r] * enc, acc[mb][nb][r + 1] * enc),
                pack_f16(acc[mb][nb][r + 2] * enc, acc[mb][nb][r + 3] * enc),
                pack_f16(acc[mb][nb][r + 4] * enc, acc[mb][nb][r + 5] * enc),
                pack_f16(acc[mb][nb][r + 6] * enc, acc[mb][nb][r + 7] * enc));
          }
        }
    }
  } else {
    // other rotary widths: the generic f32 partials, read by smla_combine
    float* part = a.ws + ((size_t)t * ns + split) * partial_floats_d(a.h_q, D);
    float* pm = part + (size_t)HP * D;
    float* pl = pm + HP;
    if (tid < a.h_q) {
      pm[tid] = maxx[tid];
      pl[tid] = lsum[tid] + lsum[HP + tid];
    }
    if (te > tb) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int h = 32 * mb + lrow;
        if (h < a.h_q) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              part[(size_t)h * D + d0 + 32 * nb + 8 * (i >> 2) + 4 * lhalf + (i & 3)] = acc[mb][nb][i];
        }
      }
    }
  }
}

// Scheduling order of the persistent kernel's items when there are more items than
// workgroups and one split per token: tokens by descending tile count, equal counts in
// token order (longest processing time first, so that the last items a workgroup takes
// are short ones and the workgroups finish together).  One 1024-thread workgroup takes
// the tokens 4096 at a time, four per thread (token c * 1024 + tid, c < 4): each wave
// counts, per tile count (key, capped at 63), its lanes with that key (lanes with the
// same key found by six ballots), then one scan per key over (c, wave) gives each
// token's place among the tokens of its key, and a scan over the keys (largest first)
// the key's first slot.  Above 4096 tokens a first pass builds the key histogram.
__global__ __launch_bounds__(1024) void smla_order(const int32_t* __restrict__ topk_length, int s_q, int topk,
                                                   int* __restrict__ order) {
  constexpr int NB = 64, NW = 16, CH = 4, SUPER = CH * 1024, NC = CH * NW;
  // per key: lanes of that key per (chunk, wave), then their exclusive scan (rows padded
  // to 65 words, so that the accesses below hit distinct banks)
  __shared__ int cnt[NB][NC + 1];
  __shared__ int tot[NB], off[NB], base[NB];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // the scans: thread tid serves key kb = tid / 16 (a DPP row of 16 lanes per key) and
  // its columns 4 ks .. 4 ks + 3
  const int kb = tid >> 4, ks = tid & 15;
  auto key_of = [&](int l) {
    l = l < 0 ? 0 : (l > topk ? topk : l);
    const int n = (l + T - 1) / T;
    return n < NB - 1 ? n : NB - 1;
  };
  auto dpp = [](int v, auto ctrl) {
    return __builtin_amdgcn_update_dpp(0, v, decltype(ctrl)::value, 0xF, 0xF, true);
  };
  using shr1 = std::integral_constant<int, 0x111>;
  using shr2 = std::integral_constant<int, 0x112>;
  using shr4 = std::integral_constant<int, 0x114>;
  using shr8 = std::integral_constant<int, 0x118>;
  using ror1 = std::integral_constant<int, 0x121>;
  using ror2 = std::integral_constant<int, 0x122>;
  using ror4 = std::integral_constant<int, 0x124>;
  using ror8 = std::integral_constant<int, 0x128>;
  // sum over the 16 lanes of the row, in every lane
  auto row_sum = [&](int v) {
    v += dpp(v, ror8{});
    v += dpp(v, ror4{});
    v += dpp(v, ror2{});
    v += dpp(v, ror1{});
    return v;
  };
  // off[kb] = tokens with a larger key: row kb sums tot[kb + 1 ..]
  auto key_offsets = [&]() {
    int v = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = kb + 1 + ks + 16 * r;
      if (b < NB) v += tot[b];
    }
    v = row_sum(v);
    if (ks == 0) off[kb] = v;
  };
  const bool multi = s_q > SUPER;
  if (tid < NB) {
    tot[tid] = 0;
    base[tid] = 0;
  }
  __syncthreads();
  if (multi) {
    for (int t0 = 0; t0 < s_q; t0 += SUPER) {
      const int nrem = s_q - t0;
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(topk_length + t0, (uint32_t)(nrem < SUPER ? nrem : SUPER) * 4u);
      int lraw[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        lraw[c] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(c * 1024 + tid) * 4u, 0, 0);
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c * 1024 + tid < nrem) atomicAdd(&tot[key_of(lraw[c])], 1);
    }
    __syncthreads();
    key_offsets();
  }
  for (int s0 = 0; s0 < s_q; s0 += SUPER) {
    // this pass's lengths through a range-checked buffer (tokens past the end read as
    // zero), so that the four loads go out together without branches
    const int nrem = s_q - s0;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(topk_length + s0, (uint32_t)(nrem < SUPER ? nrem : SUPER) * 4u);
    int lraw[CH], key[CH], rank[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
      lraw[c] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(c * 1024 + tid) * 4u, 0, 0);
#pragma unroll
    for (int c = 0; c < CH; ++c) cnt[kb][4 * ks + c] = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) key[c] = c * 1024 + tid < nrem ? key_of(lraw[c]) : -1;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool live = key[c] >= 0;
      unsigned long long peers = __ballot(live);
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const unsigned long long m = __ballot((key[c] >> k) & 1);
        peers &= ((key[c] >> k) & 1) ? m : ~m;
      }
      rank[c] = __popcll(peers & ((1ull << lane) - 1ull));
      if (live && rank[c] == 0) cnt[key[c]][c * NW + wv] = __popcll(peers);
    }
    __syncthreads();
    {
      // exclusive scan of row kb over its 64 columns: 4 per lane, then across the 16 lanes
      int v[4], run = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = run;
        run += cnt[kb][4 * ks + r];
      }
      int incl = run;
      incl += dpp(incl, shr1{});
      incl += dpp(incl, shr2{});
      incl += dpp(incl, shr4{});
      incl += dpp(incl, shr8{});
      const int excl = incl - run;
#pragma unroll
      for (int r = 0; r < 4; ++r) cnt[kb][4 * ks + r] = excl + v[r];
      if (ks == 15) tot[kb] = incl;
    }
    __syncthreads();
    if (!multi) {
      key_offsets();
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (key[c] >= 0) order[off[key[c]] + base[key[c]] + cnt[key[c]][c * NW + wv] + rank[c]] = s0 + c * 1024 + tid;
    if (multi) {
      __syncthreads();
      if (tid < NB) base[tid] += tot[tid];
      __syncthreads();
    }
  }
}

// Combine the splits of one (token, head): o = sum_s w_s acc_s / sum_s w_s l_s with
// w_s = 2^(m_s - M), M = max_s m_s, in split order, then the epilogue.  One memory
// round trip: every thread issues the loads of its 4 dims for all splits (16 at a
// time) together with the split statistics, and the cos / sin table is computed while
// they are in flight.  A split that read nothing has weight 0 and its accumulator
// (never written) is not used.
template <int D>
__global__ __launch_bounds__(CTHREADS) void smla_combine(KArgs a) {
  constexpr int OSTR = D + 4, MAXS = 64, SCH = 16;
  __shared__ __attribute__((aligned(16))) float o_l[OSTR];
  __shared__ __attribute__((aligned(16))) float cs[D / 2], sn[D / 2];
  __shared__ float mm[MAXS], ll[MAXS];
  const int t = blockIdx.x, h = blockIdx.y;
  const int ns = a.num_splits;
  const size_t pf = partial_floats_d(a.h_q, D);
  const float* base = a.ws + (size_t)t * ns * pf;
  const int f = threadIdx.x;  // float4 index within the head's D dims
  const bool act = f < D / 4;
  const size_t slot = (size_t)h * D + 4 * f;  // this thread's float4 of the accumulator
  float4 v[SCH];
#pragma unroll
  for (int k = 0; k < SCH; ++k)
    v[k] = (act && k < ns) ? *reinterpret_cast<const float4*>(base + (size_t)k * pf + slot)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  if ((int)threadIdx.x < ns) {
    const float* st = base + (size_t)threadIdx.x * pf + (size_t)HP * D;
    mm[threadIdx.x] = st[h];
    ll[threadIdx.x] = st[HP + h];
  }
  rope_table(a.positions[t], a, cs, sn);
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, mm[s]);
  float den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ns; s0 += SCH) {
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < SCH; ++k)
        v[k] = (act && s0 + k < ns) ? *reinterpret_cast<const float4*>(base + (size_t)(s0 + k) * pf + slot)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < SCH; ++k) {
      if (s0 + k < ns) {
        const float ms = mm[s0 + k];
        const float wv = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
        den += wv * ll[s0 + k];
        // select, never multiply: a split with weight 0 may hold an unwritten accumulator
        if (wv != 0.f) {
          num.x += wv * v[k].x;
          num.y += wv * v[k].y;
          num.z += wv * v[k].z;
          num.w += wv * v[k].w;
        }
      }
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  if (act) *reinterpret_cast<float4*>(o_l + 4 * f) = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
  __syncthreads();
  epilogue<D, CTHREADS>(o_l, OSTR, 1, h, t, a, cs, sn);
}

// Combine of smla_ws's splits for up to 8 splits per token (one round of loads): the
// partials are read in their register order so that every load instruction covers 512
// contiguous bytes per 32 threads.  Workgroup (token, y): y = 4v + 2mb + nbp selects the P.V wave v, head block
// mb and the block pair nb = 2nbp, 2nbp + 1; thread (lrow, gp, nbl) owns dims 16gp ..
// 16gp + 15 of block nb = 2nbp + nbl of head 32mb + lrow (slots g = 2gp, 2gp + 1, both
// lane halves).  Then o = sum_s w_s acc_s / sum_s w_s l_s (w_s = 2^(m_s - M), M the largest
// m_s, taken before the weights so that they do not depend on one another, the sums in
// split order; a split that read nothing has m_s = -inf and is never touched), inverse
// RoPE with the cos / sin table the splits wrote (blocks 14 and 15 are the two waves of
// the last workgroup pair: the partner values cross through LDS), the block amax over the
// thread pair (gp = 0, 1), UE8M0 exponent and E4M3 codes.
__global__ __launch_bounds__(CTHREADS) void smla_combine_lm4(KArgs a) {
  constexpr int D = 512, SCH = 8;
  __shared__ __attribute__((aligned(16))) float xch[CTHREADS * 16];
  const int t = blockIdx.x, y = blockIdx.y, v = y >> 2, mb = (y >> 1) & 1, nbp = y & 1;
  const int tid = threadIdx.x, lrow = tid & 31, gp = (tid >> 5) & 1, nbl = tid >> 6, nb = 2 * nbp + nbl;
  const int h = 32 * mb + lrow, hq = a.h_q, ns = a.num_splits;
  const size_t pf = partial_floats_d(hq, D);
  const float* base = a.ws + (size_t)t * ns * pf;
  // 16-byte slots of this thread in a split: g2 = gp, lanes lrow and lrow + 32; the
  // thread's 16 dims 16gp .. 16gp + 15 are halves 0..3 (dims 0..3), 4..7 (8..11) of the
  // first and 0..3 (4..7), 4..7 (12..15) of the second
  const int s0 = ((((v * 2 + mb) * 4 + nb) * 2 + gp) * 64) + lrow;
  const int gb = 4 * v + nb;
  const bool rot = a.rope_dim > 0 && v == 3 && nbp == 1;
  // the rotary workgroups' cos / sin of dims 16 gp .. 16 gp + 15 of the pair, written by
  // the splits (split 0's copy), loaded with the first chunk
  float4 rc[4], rs[4];
  if (rot) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rc[q] = reinterpret_cast<const float4*>(base + WSP_ROPE + 16 * gp)[q];
      rs[q] = reinterpret_cast<const float4*>(base + WSP_ROPE + 32 + 16 * gp)[q];
    }
  }
  float M = -INFINITY, den = 0.f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += SCH) {
    // every load of the chunk goes out before the first use
    uint4 x[SCH][2];
    float mv[SCH], lv[SCH], dv[SCH];
#pragma unroll
    for (int k = 0; k < SCH; ++k)
      if (c0 + k < ns) {
        const float* sp = base + (size_t)(c0 + k) * pf;
        const uint4* p4 = reinterpret_cast<const uint4*>(sp) + s0;
        x[k][0] = p4[0];
        x[k][1] = p4[32];
        dv[k] = sp[WSP_SCL + gb * HP + h];
        mv[k] = sp[WSP_M + h];
        lv[k] = sp[WSP_L + h];
      }
    // the chunk's largest m first (one rescale of the running sums per chunk), then every
    // split's weight on its own: no chain from split to split
    float Mc = M;
#pragma unroll
    for (int k = 0; k < SCH; ++k)
      if (c0 + k < ns) Mc = fmaxf(Mc, mv[k]);
    if (Mc > M) {
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
      den *= r;
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] *= r;
      M = Mc;
    }
#pragma unroll
    for (int k = 0; k < SCH; ++k)
      if (c0 + k < ns && mv[k] != -INFINITY) {
        const float wv = __builtin_amdgcn_exp2f(mv[k] - M);
        den += wv * lv[k];
        const float ws = wv * dv[k];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t xw[4] = {x[k][u].x, x[k][u].y, x[k][u].z, x[k][u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int e = 4 * u + 8 * (q >> 1) + 2 * (q & 1);
            o[e] += ws * f16_lo(xw[q]);
            o[e + 1] += ws * f16_hi(xw[q]);
          }
        }
      }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] *= inv;
  if (rot) {
    // (448 + j, 480 + j), j = 16gp + e: block 14 (nbl 0) takes o c + o' s, block 15 o c - o' s
#pragma unroll
    for (int e = 0; e < 16; ++e) xch[tid * 16 + e] = o[e];
    __syncthreads();
    const float sg = nbl ? -1.f : 1.f;
    const float cv[16] = {rc[0].x, rc[0].y, rc[0].z, rc[0].w, rc[1].x, rc[1].y, rc[1].z, rc[1].w,
                          rc[2].x, rc[2].y, rc[2].z, rc[2].w, rc[3].x, rc[3].y, rc[3].z, rc[3].w};
    const float sv[16] = {rs[0].x, rs[0].y, rs[0].z, rs[0].w, rs[1].x, rs[1].y, rs[1].z, rs[1].w,
                          rs[2].x, rs[2].y, rs[2].z, rs[2].w, rs[3].x, rs[3].y, rs[3].z, rs[3].w};
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = __builtin_fmaf(sg * xch[(tid ^ 64) * 16 + e], sv[e], o[e] * cv[e]);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o[e]));
  amax = pair_max(amax);
  if (h >= hq) return;
  const size_t g0 = ((size_t)t * hq + h) * D + 32 * gb + 16 * gp;
  const int e8 = ue8m0_exp(amax);
  const float sc = ue8m0_f32((uint32_t)e8);
  uint32_t wd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) wd[q] = enc2(enc2(0u, o[4 * q], o[4 * q + 1], sc, false), o[4 * q + 2], o[4 * q + 3], sc, true);
  *reinterpret_cast<uint4*>(a.out_fp8 + g0) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (gp == 0) a.out_scales[((size_t)t * hq + h) * (D / 32) + gb] = (uint8_t)e8;
  if (a.out_f32) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<float4*>(a.out_f32 + g0)[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  }
}

// Combine of smla_ws's splits for more than 8 splits per token, reading the partials in
// their register order.  Workgroup (token, y), y = 4v + 2mb + nbp, covers P.V wave v's blocks
// nb = 2nbp, 2nbp + 1 for the 32 heads of head block mb: 512 threads.  Wave wv holds heads
// 32mb + 4wv .. + 3 and lane (nbl, g, lhalf, lq) (bits 5, 4..3, 2, 1..0) the float4 slot
// (g, lhalf) of block nb = 2nbp + nbl of head 32mb + 4wv + lq, i.e. its dims 8g + 4lhalf ..
// + 3, so that the 8 threads of a (head, block) and the two blocks of a rotary pair share a
// wave: the block amax and the pair exchange go through DPP and lane swaps, with no LDS and
// no barrier.  A wave reads 64-byte runs of each split's partials, and every split's load
// goes out in one round (chunks of 16).  Then o = sum_s w_s acc_s / sum_s w_s l_s (w_s =
// 2^(m_s - M), M the running maximum, raised once per chunk of 16 splits before that
// chunk's weights, which then do not depend on one another; the sums in split order; a
// split that read nothing has m_s = -inf and is never touched), inverse RoPE with the
// cos / sin table the splits wrote, the UE8M0 exponent and the E4M3 codes.
constexpr int LMT = 512;  // smla_combine_lm1 threads
__global__ __launch_bounds__(LMT) void smla_combine_lm1(KArgs a) {
  constexpr int D = 512, SCH = 16;
  const int t = blockIdx.x, y = blockIdx.y, v = y >> 2, mb = (y >> 1) & 1, nbp = y & 1;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int lq = lane & 3, lhalf = (lane >> 2) & 1, g = (lane >> 3) & 3, nbl = lane >> 5;
  const int lrow = 4 * wv + lq, nb = 2 * nbp + nbl;
  const int h = 32 * mb + lrow, hq = a.h_q, ns = a.num_splits;
  const size_t pf = partial_floats_d(hq, D);
  const float* base = a.ws + (size_t)t * ns * pf;
  // registers 4g .. 4g + 3 of lane lrow + 32 lhalf of the P.V wave: half g & 1 of its
  // 16-byte slot g >> 1
  const int slot = (((((v * 2 + mb) * 4 + nb) * 2 + (g >> 1)) * 64) + lrow + 32 * lhalf) * 2 + (g & 1);  // 8-byte index
  const int gb = 4 * v + nb;
  const bool rot = a.rope_dim > 0 && v == 3 && nbp == 1;  // (uniform over the workgroup)
  // the rotary workgroups' cos / sin of pair dims 8g + 4lhalf .. + 3, written by the
  // splits (split 0's copy), loaded with the first chunk
  float4 rc = make_float4(0.f, 0.f, 0.f, 0.f), rs = rc;
  if (rot) {
    rc = *reinterpret_cast<const float4*>(base + WSP_ROPE + 8 * g + 4 * lhalf);
    rs = *reinterpret_cast<const float4*>(base + WSP_ROPE + 32 + 8 * g + 4 * lhalf);
  }
  float M = -INFINITY, den = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < ns; c0 += SCH) {
    uint2 x[SCH];
    float mv[SCH], lv[SCH], dv[SCH];
#pragma unroll
    for (int k = 0; k < SCH; ++k)
      if (c0 + k < ns) {
        const float* sp = base + (size_t)(c0 + k) * pf;
        x[k] = reinterpret_cast<const uint2*>(sp)[slot];
        dv[k] = sp[WSP_SCL + gb * HP + h];
        mv[k] = sp[WSP_M + h];
        lv[k] = sp[WSP_L + h];
      }
    // the chunk's largest m first (one rescale of the running sums per chunk), then every
    // split's weight on its own: no chain from split to split
    float Mc = M;
#pragma unroll
    for (int k = 0; k < SCH; ++k)
      if (c0 + k < ns) Mc = fmaxf(Mc, mv[k]);
    if (Mc > M) {
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
      den *= r;
      o.x *= r; o.y *= r; o.z *= r; o.w *= r;
      M = Mc;
    }
#pragma unroll
    for (int k = 0; k < SCH; ++k)
      if (c0 + k < ns && mv[k] != -INFINITY) {
        const float wv_ = __builtin_amdgcn_exp2f(mv[k] - M);
        den += wv_ * lv[k];
        const float ws = wv_ * dv[k];
        o.x += ws * f16_lo(x[k].x); o.y += ws * f16_hi(x[k].x); o.z += ws * f16_lo(x[k].y); o.w += ws * f16_hi(x[k].y);
      }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  float ov[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
  if (rot) {
    // (448 + j, 480 + j), j = 8g + 4lhalf + e: block 14 (nbl 0) takes o c + o' s, block 15
    // o c - o' s; the partner is lane l ^ 32
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = xor32_f32(ov[e]);
    const float sg = nbl ? -1.f : 1.f;
    const float cv[4] = {rc.x, rc.y, rc.z, rc.w}, sv[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = __builtin_fmaf(sg * pv[e], sv[e], ov[e] * cv[e]);
  }
  // block amax over the 8 lanes of the (head, block): bits 2..3 by two rotations within the
  // 16-lane row, bit 4 by the row swap
  float amax = fmaxf(fmaxf(fabsf(ov[0]), fabsf(ov[1])), fmaxf(fabsf(ov[2]), fabsf(ov[3])));
  amax = fmaxf(amax, dpp_perm_f32<0x124>(amax));  // row_ror:4
  amax = fmaxf(amax, dpp_perm_f32<0x128>(amax));  // row_ror:8
  amax = xor16_max(amax);
  if (h >= hq) return;
  const size_t g0 = ((size_t)t * hq + h) * D + 32 * gb + 8 * g + 4 * lhalf;
  const int e8 = ue8m0_exp(amax);
  const float sc = ue8m0_f32((uint32_t)e8);
  *reinterpret_cast<uint32_t*>(a.out_fp8 + g0) = enc2(enc2(0u, ov[0], ov[1], sc, false), ov[2], ov[3], sc, true);
  if (g == 0 && lhalf == 0) a.out_scales[((size_t)t * hq + h) * (D / 32) + gb] = (uint8_t)e8;
  if (a.out_f32) *reinterpret_cast<float4*>(a.out_f32 + g0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
}

}  // namespace

// compute units of the current device (one persistent workgroup each)
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

template <int D, int EB>
hipError_t launch_t(const LaunchArgs& x, const KArgs& k) {
  const int ns = x.num_splits;
  const int items = x.s_q * ns;
  const bool ws = D == 512 && EB == 1 && (x.rope_dim == 0 || x.rope_dim == 64);
  if (ws) {
    const int cus = device_cus();
    KArgs kw = k;
    if (ns == 1 && items > cus) {
      // more items than workgroups: take them longest first
      int* order = reinterpret_cast<int*>(k.ws);
      hipLaunchKernelGGL(smla_order, dim3(1), dim3(1024), 0, x.stream, x.topk_length, x.s_q, x.topk, order);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      kw.order = order;
    }
    if (x.ev_main) (void)hipEventRecord(x.ev_main, x.stream);
    hipLaunchKernelGGL(smla_ws, dim3((unsigned)(items < cus ? items : cus)), dim3(NTHREADS), 0, x.stream, kw);
  } else {
    if (x.ev_main) (void)hipEventRecord(x.ev_main, x.stream);
    hipLaunchKernelGGL((smla_main<D, EB>), dim3((unsigned)items), dim3(NTHREADS), 0, x.stream, k);
  }
  hipError_t e = hipGetLastError();
  if (x.ev_split) (void)hipEventRecord(x.ev_split, x.stream);
  if (e != hipSuccess || ns == 1) {
    if (x.ev_end) (void)hipEventRecord(x.ev_end, x.stream);
    return e;
  }
  if (ws)
    if (ns <= 8)
      hipLaunchKernelGGL(smla_combine_lm4, dim3((unsigned)x.s_q, 16u), dim3(CTHREADS), 0, x.stream, k);
    else
      hipLaunchKernelGGL(smla_combine_lm1, dim3((unsigned)x.s_q, 16u), dim3(LMT), 0, x.stream, k);
  else
    hipLaunchKernelGGL((smla_combine<D>), dim3((unsigned)x.s_q, (unsigned)x.h_q), dim3(CTHREADS), 0, x.stream, k);
  e = hipGetLastError();
  if (x.ev_end) (void)hipEventRecord(x.ev_end, x.stream);
  return e;
}

}  // namespace

hipError_t launch(const LaunchArgs& x) {
  const KArgs k = make_kargs(x);
  if (x.cmp_pool) {
    static_assert(NvCfg::MAX_ROPE >= kNvMaxRope, "the host's rotary limit for the two-pool kernel");
    if (x.d != 512 || x.kv_format != 0) return hipErrorInvalidValue;
    KArgs kn = k;
    if (x.num_splits == 1 && x.s_q > device_cus()) {
      // more tokens than compute units: longest first
      int* order = reinterpret_cast<int*>(k.ws);
      hipLaunchKernelGGL(smla_order, dim3(1), dim3(1024), 0, x.stream, x.topk_length, x.s_q, x.topk, order);
      const hipError_t eo = hipGetLastError();
      if (eo != hipSuccess) return eo;
      kn.order = order;
    }
    if (x.ev_main) (void)hipEventRecord(x.ev_main, x.stream);
    hipLaunchKernelGGL(smla_nv, dim3((unsigned)(x.s_q * x.num_splits)), dim3(NTHREADS), 0, x.stream, kn);
    hipError_t e = hipGetLastError();
    if (x.ev_split) (void)hipEventRecord(x.ev_split, x.stream);
    if (e == hipSuccess && x.num_splits > 1) {
      // the split partials are in smla_ws's format for rotary widths 0 and 64
      if (x.rope_dim != 0 && x.rope_dim != 64)
        hipLaunchKernelGGL((smla_combine<512>), dim3((unsigned)x.s_q, (unsigned)x.h_q), dim3(CTHREADS), 0, x.stream, k);
      else if (x.num_splits <= 8)
        hipLaunchKernelGGL(smla_combine_lm4, dim3((unsigned)x.s_q, 16u), dim3(CTHREADS), 0, x.stream, k);
      else
        hipLaunchKernelGGL(smla_combine_lm1, dim3((unsigned)x.s_q, 16u), dim3(LMT), 0, x.stream, k);
      e = hipGetLastError();
    }
    if (x.ev_end) (void)hipEventRecord(x.ev_end, x.stream);
    return e;
  }
  if (x.d == 512 && x.kv_format == 0) return launch_t<512, 1>(x, k);
  if (x.d == 128 && x.kv_format == 0) return launch_t<128, 1>(x, k);
  if (x.d == 128 && x.kv_format == 1) return launch_t<128, 2>(x, k);
  return hipErrorInvalidValue;
}

}  // namespace smla
