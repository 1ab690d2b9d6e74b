// Backward of the latent mixing steps between the down-projection and the
// attention (gfx950, HBM bound): causal sequence convolution, channel
// convolution, q-k-mean, value-shift, L2 normalisation and RoPE
// [GS-EN "2. Methodology" / Convolutional Mixing, Q-K-Mean, Value-Shift,
//  RoPE Integration; EDG "How Compressed Convolutional Attention Works"].
// Each step's derivative is the chain rule on the forward definition:
//   RoPE is a rotation per channel pair: its transpose rotates back;
//   y = m / max(|m|, eps):  dm = (dy - y <y, dy>) / |m| (|m| > eps), dy / eps;
//   q-k-mean (q += (q~ + k~_g) / 2, k += (k~ + mean_g q~) / 2): q~ collects
//     dq / 2 and dk_g / (2G), k~ collects dk / 2 and the group sum of dq / 2;
//   channel conv b[i] = sum_j w[j] a[i-j]:  da[i] = sum_j w[j] db[i+j];
//   sequence conv a[t] = sum_j w[j] u[t-j]: du[t] = sum_j w[j] da[t+j];
//   value-shift: the shifted heads' token t feeds token t+1.
//
// Design (MI355X): two passes over fp32 activations.
//  * head pass: one d-lane segment per (token, q or k head) recomputes the
//    forward from the fp32 down-projection output (sequence and channel conv,
//    q-k-mean, norm, rotation) and runs the per-head backward (RoPE, norm,
//    channel conv): channel neighbours and pair partners are lane shuffles,
//    the norms segment reductions.  It writes dm (the mixed q/k cotangent)
//    and da (the sequence conv output's cotangent), plus per-(token, head)
//    partial sums of the channel-tap and temperature gradients.
//  * channel pass: one thread per (channel, 16-token run) combines the
//    sequence-conv transpose (reads da at t .. t+k_s-1), the q-k-mean skip
//    terms and the value-shift into dz, the cotangent of the down-projection
//    output, and accumulates its sequence-tap gradient over the run.
//  * tap / temperature gradients: deterministic two-level column sums.
#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

template <int D>
__global__ __launch_bounds__(256) void mix_bwd_head_kernel(MixShape s, MixTaps w,
                                                           const float *__restrict__ qkv,
                                                           const float *__restrict__ gq,
                                                           const float *__restrict__ dk,
                                                           float *__restrict__ dm_out,
                                                           float *__restrict__ da_out,
                                                           float *__restrict__ tau_part,
                                                           float *__restrict__ chan_part) {
  constexpr int SEG = D < 64 ? D : 64;      // lanes per (token, head)
  constexpr int CPL = D / SEG;              // channels per lane (1, or 2 at d = 128)
  constexpr int UPW = 64 / SEG;             // units per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % SEG, sbase = lane - li;
  const int H = s.Hq + s.Hkv;
  const long long unit = ((long long)blockIdx.x * 4 + wave) * UPW + lane / SEG;
  const bool active = unit < (long long)s.B * s.T * H;
  const long long bt = active ? unit / H : 0;
  const int hh = active ? (int)(unit % H) : 0;
  const int b = (int)(bt / s.T), t = (int)(bt % s.T);
  const bool is_q = hh < s.Hq;
  const int g = is_q ? hh / s.G : hh - s.Hq;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int colbase = is_q ? hh * D : eq + g * D;          // in the qkv row and in dm / da rows
  const float *seqw = is_q ? w.q_seq + (size_t)hh * D * s.ks : w.k_seq + (size_t)g * D * s.ks;
  const float *chw = is_q ? w.q_chan + (size_t)hh * s.kc : w.k_chan + (size_t)g * s.kc;
  const float *row_t = qkv + ((size_t)b * s.T + t) * N;

  // every global read first, so that they are in flight together: the
  // k_s pre-conv rows (zero before the sequence start), the skip terms of
  // q-k-mean, the taps and the incoming cotangent
  float cw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cw[j] = chw[min(j, s.kc - 1)];
  float uv[CPL][4], wsv[CPL][4], skip[CPL], gin[CPL];
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    const int i = li + SEG * p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uv[p][j] = qkv[((size_t)b * s.T + max(t - j, 0)) * N + colbase + i];
      wsv[p][j] = seqw[i * s.ks + min(j, s.ks - 1)];
    }
    if (is_q) {
      skip[p] = row_t[eq + g * D + i];
      gin[p] = gq[((size_t)b * s.T + t) * eq + hh * D + i];
    } else {
      float qs = 0.f;
      for (int h2 = 0; h2 < s.G; ++h2) qs += row_t[(g * s.G + h2) * D + i];
      skip[p] = qs * (1.f / (float)s.G);
      gin[p] = dk[((size_t)b * s.T + t) * ekv + g * D + i];
    }
  }
  const float tau_h = is_q ? w.tau[hh] : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j >= s.kc) cw[j] = 0.f;
#pragma unroll
    for (int p = 0; p < CPL; ++p)
      if (j >= s.ks || t - j < 0) wsv[p][j] = 0.f;
  }

  // channel i of this lane's p-th slot is li + SEG * p
  float a[CPL], m[CPL];
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += wsv[p][j] * uv[p][j];
    a[p] = acc;
  }
  // value of `v` (slots v[0..CPL)) at channel ci of this segment (0 outside [0, D))
  auto at = [&](const float (&v)[CPL], int ci) {
    const int cc = ci < 0 ? 0 : (ci >= D ? D - 1 : ci);
    const int src = sbase + cc % SEG, pp = cc / SEG;
    float r = __shfl(v[0], src, 64);
    if constexpr (CPL == 2) {
      const float r1 = __shfl(v[1], src, 64);
      r = pp ? r1 : r;
    }
    return (ci < 0 || ci >= D) ? 0.f : r;
  };
  auto seg_sum = [&](float v) {
#pragma unroll
    for (int o = 1; o < SEG; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
  };

  // forward recompute: channel conv, q-k-mean, norm
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    const int i = li + SEG * p;
    float bb = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) bb += cw[j] * at(a, i - j);
    if (s.use_mean) bb += 0.5f * (uv[p][0] + skip[p]);
    m[p] = bb;
  }
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < CPL; ++p) ss += m[p] * m[p];
  const float nrm = sqrtf(seg_sum(ss));
  const bool big = nrm > s.eps;
  const float inv = s.use_norm ? 1.f / (big ? nrm : s.eps) : 1.f;
  float n[CPL];
#pragma unroll
  for (int p = 0; p < CPL; ++p) n[p] = m[p] * inv;

  // cotangent of the rotated vector, rotation back, temperature partial
  float dn[CPL];
  float tau_acc = 0.f;
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    const int i = li + SEG * p;
    const float2 cs = rope_cs_theta(t, s.theta[i >> 1], s.rope_base);
    const float dr = is_q ? tau_h * gin[p] : gin[p];
    if (is_q) {
      // the rotated, normalised q this lane holds: <r, g> summed below
      const float partner = __shfl_xor(n[p], 1, 64);
      const float r = (i & 1) ? partner * cs.y + n[p] * cs.x : n[p] * cs.x - partner * cs.y;
      tau_acc += r * gin[p];
    }
    const float dpartner = __shfl_xor(dr, 1, 64);
    // pair (x0, x1) -> (x0 c - x1 s, x0 s + x1 c); transpose: (g0 c + g1 s, -g0 s + g1 c)
    dn[p] = (i & 1) ? -dpartner * cs.y + dr * cs.x : dr * cs.x + dpartner * cs.y;
  }
  const float tau_sum = seg_sum(tau_acc);

  // norm backward
  float dm[CPL];
  if (s.use_norm) {
    float nd = 0.f;
#pragma unroll
    for (int p = 0; p < CPL; ++p) nd += n[p] * dn[p];
    nd = seg_sum(nd);
#pragma unroll
    for (int p = 0; p < CPL; ++p) dm[p] = big ? (dn[p] - n[p] * nd) / nrm : dn[p] / s.eps;
  } else {
#pragma unroll
    for (int p = 0; p < CPL; ++p) dm[p] = dn[p];
  }

  // channel conv backward and its tap partials
  float da[CPL];
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    const int i = li + SEG * p;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += cw[j] * at(dm, i + j);
    da[p] = acc;
  }
  float cpart[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < CPL; ++p) acc += dm[p] * at(a, li + SEG * p - j);
    cpart[j] = seg_sum(acc);
  }

  if (!active) return;
  const int wcols = eq + ekv;
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    const int i = li + SEG * p;
    const size_t o = (size_t)bt * wcols + (is_q ? hh * D : eq + g * D) + i;
    dm_out[o] = dm[p];
    da_out[o] = da[p];
  }
  if (li == 0) {
    if (is_q) tau_part[(size_t)bt * s.Hq + hh] = tau_sum;
    for (int j = 0; j < s.kc; ++j) chan_part[((size_t)bt * H + hh) * s.kc + j] = cpart[j];
  }
}

// Tokens per thread of the channel pass.
static constexpr int MIX_BWD_TB = 16;

template <typename TZ>
__global__ __launch_bounds__(256) void mix_bwd_chan_kernel(MixShape s, MixTaps w,
                                                           const float *__restrict__ qkv,
                                                           const float *__restrict__ dm,
                                                           const float *__restrict__ da,
                                                           const float *__restrict__ dv,
                                                           TZ *__restrict__ dz,
                                                           float *__restrict__ seq_part) {
  const int D = s.d;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv, wcols = eq + ekv;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int ntb = (s.T + MIX_BWD_TB - 1) / MIX_BWD_TB;
  const int b = blockIdx.y / ntb, tb = blockIdx.y % ntb;
  const int tbeg = tb * MIX_BWD_TB, tend = min(s.T, tbeg + MIX_BWD_TB);
  if (c >= N) return;
  const size_t rb = (size_t)b * s.T;
  if (c < wcols) {
    const bool is_q = c < eq;
    const int i = (is_q ? c : c - eq) % D;
    const int g = is_q ? (c / D) / s.G : (c - eq) / D;
    const float *seqw = is_q ? w.q_seq + (size_t)c * s.ks : w.k_seq + (size_t)(c - eq) * s.ks;
    float ws[4], dws[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ws[j] = j < s.ks ? seqw[j] : 0.f;
      dws[j] = 0.f;
    }
    // rolling windows: dwin[j] = da[t + j], uwin[j] = u[t - j] (zero outside [0, T))
    float dwin[4], uwin[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dwin[j] = (j < s.ks && tbeg + j < s.T) ? da[(rb + tbeg + j) * wcols + c] : 0.f;
      uwin[j] = (j < s.ks && tbeg - j >= 0) ? qkv[(rb + tbeg - j) * N + c] : 0.f;
    }
    for (int t = tbeg; t < tend; ++t) {
      const float nxt_d = (t + s.ks < s.T) ? da[(rb + t + s.ks) * wcols + c] : 0.f;
      const float nxt_u = (t + 1 < s.T) ? qkv[(rb + t + 1) * N + c] : 0.f;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += ws[j] * dwin[j];
      if (s.use_mean) {
        const float *dmr = dm + (rb + t) * wcols;
        if (is_q) {
          acc += 0.5f * dmr[c] + (0.5f / (float)s.G) * dmr[eq + g * D + i];
        } else {
          float qsum = 0.f;
          for (int h2 = 0; h2 < s.G; ++h2) qsum += dmr[(g * s.G + h2) * D + i];
          acc += 0.5f * (dmr[c] + qsum);
        }
      }
      dz[(rb + t) * N + c] = from_f32<TZ>(acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) dws[j] += dwin[0] * uwin[j];
      // slide: window entries j >= ks stay zero (their taps are zero too)
#pragma unroll
      for (int j = 0; j < 3; ++j) dwin[j] = dwin[j + 1];
      dwin[3] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == s.ks - 1) dwin[j] = nxt_d;
#pragma unroll
      for (int j = 3; j > 0; --j) uwin[j] = uwin[j - 1];
      uwin[0] = nxt_u;
    }
    float *dst = seq_part + ((size_t)b * ntb + tb) * wcols * s.ks + (size_t)c * s.ks;
    for (int j = 0; j < s.ks; ++j) dst[j] = dws[j];
  } else {
    const int cv = c - wcols, gv = cv / D;
    const int shift = (s.use_shift && gv >= s.Hkv / 2) ? 1 : 0;
    for (int t = tbeg; t < tend; ++t) {
      const int src = t + shift;
      const float v = src < s.T ? dv[(rb + src) * ekv + cv] : 0.f;
      dz[(rb + t) * N + c] = from_f32<TZ>(v);
    }
  }
}

// out[rb * ncols + j] = sum of in[r * C + col0 + j] over the rows r of row
// block rb (rows_per_block rows), j < ncols: 64 columns per workgroup, four
// row phases reduced through LDS; fixed order, so the sums are deterministic.
__global__ __launch_bounds__(256) void colsum_kernel(const float *__restrict__ in, long long R,
                                                     int C, int col0, int ncols,
                                                     int rows_per_block, float *__restrict__ out) {
  __shared__ float red[4][64];
  const int cl = threadIdx.x % 64, rs = threadIdx.x / 64;
  const int j = blockIdx.x * 64 + cl;
  const long long r0 = (long long)blockIdx.y * rows_per_block;
  const long long r1 = min(R, r0 + rows_per_block);
  float acc = 0.f;
  if (j < ncols)
    for (long long r = r0 + rs; r < r1; r += 4) acc += in[r * C + col0 + j];
  red[rs][cl] = acc;
  __syncthreads();
  if (rs == 0 && j < ncols)
    out[(size_t)blockIdx.y * ncols + j] = (red[0][cl] + red[1][cl]) + (red[2][cl] + red[3][cl]);
}

// Column sums of in [R][C] (columns col0 .. col0 + ncols) into out[ncols]:
// blocks of 64 rows, then one block over the block sums.
static hipError_t colsum(const float *in, long long R, int C, int col0, int ncols, float *blk,
                         float *out, hipStream_t stream) {
  const unsigned cb = (unsigned)((ncols + 63) / 64);
  const long long nblk = (R + 63) / 64;
  hipLaunchKernelGGL(colsum_kernel, dim3(cb, (unsigned)nblk), dim3(256), 0, stream, in, R, C, col0,
                     ncols, 64, blk);
  hipLaunchKernelGGL(colsum_kernel, dim3(cb, 1), dim3(256), 0, stream, blk, nblk, ncols, 0, ncols,
                     (int)nblk, out);
  return hipGetLastError();
}

size_t mix_backward_scratch_floats(const MixShape &s) {
  const size_t BT = (size_t)s.B * s.T;
  const int H = s.Hq + s.Hkv;
  const int ntb = (s.T + MIX_BWD_TB - 1) / MIX_BWD_TB;
  const size_t wcols = (size_t)(s.Hq + s.Hkv) * s.d;
  const size_t seq_rows = (size_t)s.B * ntb, seq_cols = wcols * s.ks;
  const size_t blk = ((BT + 63) / 64) * (size_t)(H * s.kc > s.Hq ? H * s.kc : s.Hq);
  const size_t blk_seq = ((seq_rows + 63) / 64) * seq_cols;
  // tau partials, channel-tap partials, seq-tap partials, row-block sums
  return BT * s.Hq + BT * H * s.kc + seq_rows * seq_cols + (blk > blk_seq ? blk : blk_seq);
}

template <typename TZ>
hipError_t launch_mix_backward(const MixShape &s, const MixTaps &w, const MixBwdArgs<TZ> &a,
                               hipStream_t stream) {
  const long long units = (long long)s.B * s.T * (s.Hq + s.Hkv);
  const int seg = s.d < 64 ? s.d : 64;
  const long long per_wg = 4LL * (64 / seg);
  const unsigned nwg = (unsigned)((units + per_wg - 1) / per_wg);
  const size_t BT = (size_t)s.B * s.T;
  const int H = s.Hq + s.Hkv;
  const int ntb = (s.T + MIX_BWD_TB - 1) / MIX_BWD_TB;
  const int wcols = (s.Hq + s.Hkv) * s.d, N = wcols + s.Hkv * s.d;
  const int eq = s.Hq * s.d, ekv = s.Hkv * s.d;
  float *tau_part = a.scratch;
  float *chan_part = tau_part + BT * s.Hq;
  float *seq_part = chan_part + BT * H * s.kc;
  float *blk = seq_part + (size_t)s.B * ntb * wcols * s.ks;

  switch (s.d) {
    case 16: hipLaunchKernelGGL((mix_bwd_head_kernel<16>), dim3(nwg), dim3(256), 0, stream, s, w, a.qkv, a.gq, a.dk, a.dm, a.da, tau_part, chan_part); break;
    case 32: hipLaunchKernelGGL((mix_bwd_head_kernel<32>), dim3(nwg), dim3(256), 0, stream, s, w, a.qkv, a.gq, a.dk, a.dm, a.da, tau_part, chan_part); break;
    case 64: hipLaunchKernelGGL((mix_bwd_head_kernel<64>), dim3(nwg), dim3(256), 0, stream, s, w, a.qkv, a.gq, a.dk, a.dm, a.da, tau_part, chan_part); break;
    case 128: hipLaunchKernelGGL((mix_bwd_head_kernel<128>), dim3(nwg), dim3(256), 0, stream, s, w, a.qkv, a.gq, a.dk, a.dm, a.da, tau_part, chan_part); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mix_bwd_chan_kernel<TZ>), dim3((N + 255) / 256, s.B * ntb), dim3(256), 0,
                     stream, s, w, a.qkv, a.dm, a.da, a.dv, a.dz, seq_part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // temperature [BT][Hq]; channel taps [BT][H * kc] (q heads, then k heads);
  // sequence taps [B * ntb][(e_q + e_kv) * ks] (q channels, then k channels).
  // The row-block scratch is reused: each colsum finishes before the next
  // one starts on the same stream.
  if ((e = colsum(tau_part, (long long)BT, s.Hq, 0, s.Hq, blk, a.d_tau, stream)) != hipSuccess) return e;
  if ((e = colsum(chan_part, (long long)BT, H * s.kc, 0, s.Hq * s.kc, blk, a.d_q_chan, stream)) != hipSuccess) return e;
  if ((e = colsum(chan_part, (long long)BT, H * s.kc, s.Hq * s.kc, s.Hkv * s.kc, blk, a.d_k_chan, stream)) != hipSuccess) return e;
  if ((e = colsum(seq_part, (long long)s.B * ntb, wcols * s.ks, 0, eq * s.ks, blk, a.d_q_seq, stream)) != hipSuccess) return e;
  return colsum(seq_part, (long long)s.B * ntb, wcols * s.ks, eq * s.ks, ekv * s.ks, blk, a.d_k_seq, stream);
}

template hipError_t launch_mix_backward<bf16>(const MixShape &, const MixTaps &,
                                              const MixBwdArgs<bf16> &, hipStream_t);
template hipError_t launch_mix_backward<float>(const MixShape &, const MixTaps &,
                                               const MixBwdArgs<float> &, hipStream_t);

}  // namespace cca
