// Internal definitions shared by the host calibration code and the HIP kernels:
// the codebook object, the per-head device blob and error reporting.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/aatc.h"

namespace aatc {

constexpr int kTile = 64;        // token slots per tile
constexpr int kMaxD = 128;       // largest head_dim
constexpr int kMaxFields = 384;  // fields of one record: <= d channels + 2 per record byte
constexpr int kMaxQM = 16;       // score MFMAs per token group (<= 32 words x 8 fields / 16)
constexpr int kMaxVB = 24;       // value column blocks of 16 fields per head
constexpr int kKeyAlign = 32;    // key bits per token are a multiple of one 32-bit word
constexpr int kMaxRecordBytes = kMaxD;  // bytes of one record (at most 8 bits per channel)
constexpr int kVqDim = 4;        // key coefficients per vector-quantized group
constexpr int kVqSize = 256;     // codewords per group (one index byte)
constexpr int kMaxVqGroups = kMaxD / kVqDim;

// One byte-aligned field of a token record: code bits [shift, shift + width) of channel
// chan at bits [pos, pos + width) of record byte `byte` (never crossing a byte).
struct Field {
    int chan;
    int width;
    int shift;
    int byte;
    int pos;
};

struct HeadCB {
    std::vector<double> UK, UV;      // d*d, U[i*d + j] = component i of basis vector j
    std::vector<double> lamK, lamV;  // eigenvalues (descending) or empty
    std::vector<double> muK, muV;
    std::vector<double> xK, xV;      // channel weights (empty if not calibrated)
    std::vector<int32_t> bK, bV;
    std::vector<float> stepK, stepV;
    double theta = 0.0;
    // vector-quantized keys (vq_groups > 0; bK all zero then): channels [g*4 + k],
    // weighted-domain scales s_j [d], codewords [g][256][4]
    int vq_groups = 0;
    std::vector<int32_t> vq_chan;
    std::vector<float> vq_scale, vq_cent;
    // derived: record fields sorted by (byte, pos)
    std::vector<Field> fK, fV;
    int BK = 0, BV = 0;
};

// Device blob of one head.  Arrays are sized for d = 128 and indexed densely for the
// actual d (e.g. UK[i*d + j]).
struct alignas(256) DevHead {
    int32_t d, BK, BV, nfK, nfV;
    int32_t vq_groups;  // > 0: vector-quantized keys (the vq_* arrays below)
    // encoder basis terms: 2 (W = hi + lo) or 3 (+ mid, for rates above 6.5 bits/element,
    // where the channels' cells are narrow enough that the hi + lo rounding would flip more
    // than 1e-4 of the codes)
    int32_t enc_terms;
    int32_t pad0[57];
    float UK[kMaxD * kMaxD];      // fp32 basis (query transform)
    float UV[kMaxD * kMaxD];      // fp32 basis (inverse transform of values)
    float UVt[kMaxD * kMaxD];     // its transpose, UVt[j*d + i] = UV[i*d + j]
    // Encoder bases W = U diag(1/step) (the quantizer's scale folded into the projection;
    // zero columns for uncoded channels), bf16 split, channel-major: EKt_hi[j*d + i] +
    // EKt_lo[j*d + i] = fp32(U_K[i][j] * invK[j]) (+ rounding), the MFMA operand order (16
    // consecutive bytes along i)
    uint16_t EKt_hi[kMaxD * kMaxD];
    uint16_t EKt_lo[kMaxD * kMaxD];
    uint16_t EVt_hi[kMaxD * kMaxD];
    uint16_t EVt_lo[kMaxD * kMaxD];
    uint16_t EKt_mid[kMaxD * kMaxD];  // third terms: bf16(W - hi - lo) (zero when enc_terms = 2)
    uint16_t EVt_mid[kMaxD * kMaxD];
    // query transform q' = T_K^{-1} q (T_K the key basis; T_K^{-1} = U_K^T for the KLT),
    // bf16 split in the same layout: QKt_hi[j*d + i] + QKt_lo[j*d + i] = (T_K^{-1})[j][i]
    uint16_t QKt_hi[kMaxD * kMaxD];
    uint16_t QKt_lo[kMaxD * kMaxD];
    float muV[kMaxD];
    float muK[kMaxD];
    float obias[kMaxD];           // mu_V - U_V (step_V * (2^(b-1) - 1/2)): output of all-zero codes
    // encoder accumulator start: 2^(b-1) - 1/2 - mu_K (W_hi + W_lo), fp64 sum rounded once
    // (0 for uncoded channels), so that the projection yields t + 2^(b-1) - 1/2
    float estartK[kMaxD];
    float estartV[kMaxD];
    float stepK[kMaxD], stepV[kMaxD];
    float invK[kMaxD], invV[kMaxD];
    int32_t bitsK[kMaxD], bitsV[kMaxD];
    // Encoder tables (likewise for values).  Record fields by channel: channel j's fields,
    // lowest code bits first, are cpieceK[cfirstK[j] .. cfirstK[j + 1]), each byte | pos << 8 |
    // width << 12 | shift << 16.  encpermK: the channel order of the encoder's MFMA columns
    // (position 16 k + c of block k holds channel encpermK[16 k + c]): the channels of one
    // 16-column block have first fields in record bytes distinct mod 16 where possible, so
    // that their codes land in distinct LDS banks of the staged block.
    uint32_t cpieceK[kMaxFields];
    uint32_t cpieceV[kMaxFields];
    int16_t cfirstK[kMaxD + 8];
    int16_t cfirstV[kMaxD + 8];
    uint8_t encpermK[kMaxD];
    uint8_t encpermV[kMaxD];
    // ---- decode schedule -------------------------------------------------------------
    // Score MFMAs: nqm per token group.  The B operand of lane group g (lanes 16g..16g+15,
    // K-slots 16g..16g+15) in MFMA m is four dwords; dword i is key-record word w_i of the
    // lane's token ANDed with a mask that keeps one field per byte.  kq_sched[m][g] holds
    // the four tile byte offsets 256 w_i (the record word of slots 4c..4c+3 for a lane's
    // token column c sits at 256 w_i + 16 c) and then the four masks.  kq_slot[m][g][4i+b]
    // describes the field kept in byte b: chan | shift << 8 | pos << 11 | flip << 14 (pos =
    // bit position in the byte; flip = the field ends at bit 7, so the stored inverted bit 7
    // makes the byte read 128 low), 0xFFFF for an empty byte.
    int32_t nqm;
    int32_t nvb;  // value column blocks of 16 fields
    int32_t pad1[6];
    uint32_t kq_sched[kMaxQM][4][8];
    uint16_t kq_slot[kMaxQM][4][16];
    // per key channel: the largest slot weight 2^(shift - pos) of its fields (0 if uncoded)
    float kq_fmax[kMaxD];
    // Value MFMAs: column c of block cb is value field 16 cb + c (fieldV order):
    // vb_col = (value-block offset 64 * byte of its record byte's plane) | mask << 16, the
    // field mask within the byte; padding columns are 0.
    uint32_t vb_col[kMaxVB][16];
    // Value channel j: the columns of its fields (at most 8: a field has at least one bit),
    // each col | (shift - pos + 8) << 9 | flip << 13, unused entries 0xFFFF.
    uint16_t vch[kMaxD][8];
    // ---- vector-quantized keys ---------------------------------------------------------
    // group g codes channels vq_chan[g][0..3]; its index is key-record byte g; coefficient
    // u = fp32(c * vq_scale[j]) is matched against vq_cent[g][i][0..3]; the reconstructed
    // coefficient is codeword * vq_rscale[j] (fp32 of 1 / scale).
    uint8_t vq_chan[kMaxVqGroups][kVqDim];
    float vq_scale[kMaxD];
    float vq_rscale[kMaxD];
    float vq_cent[kMaxVqGroups][kVqSize][kVqDim];
};

}  // namespace aatc

namespace aatc {
// encoder basis terms for a codebook of total_bits per token and kv-head at head_dim d:
// three above 6.5 bits/element
inline int enc_terms_for(int total_bits, int d) { return total_bits > 13 * d ? 3 : 2; }
}  // namespace aatc

struct aatc_codebook {
    int d = 0, n_layers = 0, n_kv = 0, group = 0;
    int total_bits = 0;
    double avg_bits = 0.0;
    int max_bits = 8;
    int joint = 1;
    std::vector<aatc::HeadCB> heads;
    std::vector<aatc::DevHead> blob;  // built by aatc::finalize
};

namespace aatc {

int set_error(int code, const char* fmt, ...);
int finalize(aatc_codebook* cb);  // fields, B, device blob; validates budget
uint16_t f32_to_bf16(float f);
float bf16_to_f32(uint16_t h);

}  // namespace aatc
