// LDS plan of the fused chunked kernel, shared by the kernel and the host
// launcher (which sizes the dynamic LDS and rejects shapes that do not fit).
#pragma once

#include <stddef.h>

namespace kda {

// OpBytes: 2 (fp16 MFMA operands, bf16 activations) or 4 (fp32 operands).
// CM: largest chunk the instantiation handles (32 or 64).
// DVS: value columns owned by one workgroup.
template <int DK, int DVS, int CM, int OpBytes>
struct ChunkLayout {
  static constexpr int PAD = 16 / OpBytes;        // 16-byte row padding
  static constexpr int LDK = DK + PAD;            // row stride of [CM][DK] operand tiles
  static constexpr int LC = CM + PAD;             // row stride of [*][CM] operand tiles
  static constexpr int LF = CM + 4;               // row stride of fp32 [CM][CM] tiles
  static constexpr int NB = CM / 16;

  static constexpr size_t kRowTile = size_t(CM) * LDK * OpBytes;   // [CM][DK]
  static constexpr size_t kColTile = size_t(DK) * LC * OpBytes;    // [DK][CM]
  static constexpr size_t kVT = size_t(DVS) * LC * OpBytes;         // [DVS][CM]
  static constexpr size_t kCC = size_t(CM) * LC * OpBytes;          // [CM][CM] operand
  static constexpr size_t kF32CC = size_t(CM) * LF * 4;             // [CM][CM] fp32
  static constexpr size_t kKinv = size_t(CM) * LDK * (OpBytes == 2 ? 2 : 4);

  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t a) { return (a + 255) & ~size_t(255); }

  // Regions, in order.  Live ranges within one chunk step:
  //   Q   q tile (raw, or decayed in per-channel mode)         load .. output
  //   KT  k^T (raw, or k*exp(Gx) transposed)                    load .. state update / W
  //   VT  v^T of this workgroup's value columns                 load .. U
  //   P   masked decayed q k^T                                  Gram .. output
  //   RA  k tile (load .. Gram)  |  fp32 inverse T (inverse)
  //   RB  fp32 A (Gram .. inverse)  |  -W (W .. state step)
  //   RC  per-channel Gram factors (load .. Gram)  |  T-derived operands Tw, Tu (inverse .. state step)
  //   KF  per-channel: staged gate (load) | (k*F)^T (load .. state update)
  static constexpr size_t oQ = 0;
  static constexpr size_t oKT = al(oQ + kRowTile);
  static constexpr size_t oVT = al(oKT + kColTile);
  static constexpr size_t oP = al(oVT + kVT);
  static constexpr size_t oRA = al(oP + kCC);
  static constexpr size_t oRB = al(oRA + mx(kRowTile, kF32CC));
  static constexpr size_t oRC = al(oRB + mx(kF32CC, kRowTile));
  static constexpr size_t szRC(bool ch) { return mx(ch ? kRowTile + kKinv : 0, 2 * kCC); }
  static constexpr size_t oKF(bool ch) { return al(oRC + szRC(ch)); }
  static constexpr size_t szKF(bool ch) { return ch ? mx(kColTile, size_t(CM) * DK * OpBytes) : 0; }
  // fp32 vectors
  static constexpr int kVecRows = 8;              // sq sk bt Gi Ge eG eGx eF  (each CM)
  // D[i][j] is needed for i - j >= 2 only
  static constexpr int ND = NB >= 3 ? (NB - 2) * (NB - 1) / 2 : 1;
  static constexpr int dslot(int i, int j) { return (i - 2) * (i - 1) / 2 + j; }
  static constexpr int kChanVecs = 3 * NB + ND + 1;   // tau[NB] Cb[NB] rsq[NB] D[ND] decC
  static constexpr size_t oVec(bool ch) { return al(oKF(ch) + szKF(ch)); }
  static constexpr size_t szVec(bool ch) {
    return size_t(kVecRows) * CM * 4 + 64 + (ch ? size_t(kChanVecs) * DK * 4 : 0);
  }
  static constexpr size_t bytes(bool ch) { return al(oVec(ch) + szVec(ch)); }
};

constexpr size_t kMaxLds = 160 * 1024;

}  // namespace kda
