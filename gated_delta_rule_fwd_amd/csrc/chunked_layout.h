// LDS plan of the fused chunked kernel, shared by the kernel and the host
// launcher (which sizes the dynamic LDS and rejects shapes that do not fit).
#pragma once

#include <stddef.h>

namespace kda {

// OpBytes: 2 (fp16 MFMA operands, bf16 activations) or 4 (fp32 operands).
// C: chunk size (16, 32 or 64).  DVS: value columns owned by one workgroup.
template <int DK, int DVS, int C, int OpBytes>
struct ChunkLayout {
  static constexpr int NB = C / 16;                 // 16-token blocks per chunk
  static constexpr int NCOL = C < 32 ? 32 : C;      // token columns read by 32-wide k steps
  static constexpr int PAD = 16 / OpBytes;          // 16-byte row padding
  static constexpr int LDK = DK + PAD;              // row stride of [C][DK] operand tiles
  static constexpr int LDV = DVS + PAD;             // row stride of the [C][DVS] value tile
  static constexpr int LC = NCOL + PAD;             // row stride of [C][tokens] operand tiles
  static constexpr int LF = C + 4;                  // row stride of fp32 [C][C] tiles
  static constexpr int KinvBytes = OpBytes == 2 ? 2 : 4;

  static constexpr size_t kRowTile = size_t(C) * LDK * OpBytes;     // [C][DK]
  static constexpr size_t kVTile = size_t(C) * LDV * OpBytes;        // [C][DVS]
  static constexpr size_t kCC = size_t(C) * LC * OpBytes;            // [C][tokens] operand
  static constexpr size_t kF32CC = size_t(C) * LF * 4;               // [C][C] fp32
  static constexpr size_t kGst = size_t(C) * DK * OpBytes;           // staged per-channel gate

  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t a) { return (a + 255) & ~size_t(255); }

  // Regions and what they hold within one chunk step (all tiles row-major,
  // one row per token):
  //   Q    q normalised (per-channel: and decayed)                load .. output
  //   K    k normalised (per-channel: and decayed)                load .. state step
  //   V    v, this workgroup's value columns                       load .. state step
  //   P    masked decayed q k^T                                    Gram .. output
  //   AM   fp32 A (Gram .. inverse); per-channel: staged gate first (load)
  //   RA   per-channel Gram factors Kb, Kinv (load .. Gram)  |  fp32 T and T diag(beta)
  //   KF   per-channel: k normalised and decayed to the chunk end  (load .. state update)
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = al(oQ + kRowTile);
  static constexpr size_t oV = al(oK + kRowTile);
  static constexpr size_t oP = al(oV + kVTile);
  static constexpr size_t oAM = al(oP + kCC);
  static constexpr size_t oRA = al(oAM + mx(kF32CC, kGst));
  static constexpr size_t oTu = al(oRA + kF32CC);                     // T diag(beta)
  static constexpr size_t oKinv = al(oRA + kRowTile);                 // after Kb
  static constexpr size_t szRA(bool ch) {
    return mx(ch ? (oKinv - oRA) + size_t(C) * LDK * KinvBytes : 0, (oTu - oRA) + kCC);
  }
  static constexpr size_t oKF(bool ch) { return al(oRA + szRA(ch)); }
  static constexpr size_t szKF(bool ch) { return ch ? kRowTile : 0; }
  // D[i][j] (decay of the blocks strictly between j and i) is needed for i - j >= 2
  static constexpr int ND = NB >= 3 ? (NB - 2) * (NB - 1) / 2 : 1;
  static constexpr int dslot(int i, int j) { return (i - 2) * (i - 1) / 2 + j; }
  // fp32 vectors: bt Gi Ge eG eGx eF (each C), misc[16]; per-channel:
  // tau[NB] Cb[NB] rsq[NB] D[ND] decC  (each DK)
  static constexpr int kVecRows = 6;
  static constexpr int kChanVecs = 3 * NB + ND + 1;
  static constexpr size_t oVec(bool ch) { return al(oKF(ch) + szKF(ch)); }
  static constexpr size_t szVec(bool ch) {
    return size_t(kVecRows) * C * 4 + 64 + (ch ? size_t(kChanVecs) * DK * 4 : 0);
  }
  static constexpr size_t bytes(bool ch) { return al(oVec(ch) + szVec(ch)); }
};

constexpr size_t kMaxLds = 160 * 1024;

}  // namespace kda
