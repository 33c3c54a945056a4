// Fused exact attention forward, four-wave form, for gfx950.
//
// Same method as the other forward kernels (the online-softmax forward of
// "解析 FlashAttention（4）：FlashAttention-v2", section 四, with the running
// state of "分块 Attention：重建概率，累计梯度", section 01), with a different
// division of the work:
//  * one wave per SIMD (four per workgroup) and 64 query rows per wave, as two
//    32-row blocks b0 and b1.  Every K operand read from LDS feeds the S^T
//    MFMAs of both blocks, so K costs half the LDS reads per MFMA of the
//    eight-wave forms.
//  * a wave may then hold 512 registers.  The O accumulators of both blocks
//    (128 registers) live in fixed accumulation registers (AGPRs a0-a127,
//    block (qb, db) in a[16 (qb DB + db) .. +15]) that only inline assembly
//    touches: the P V MFMAs, the rare rescale and the epilogue.  Scores, Q
//    and P stay in ordinary VGPRs under the compiler.
//  * inside one wave, key tile j runs as
//      phase 1:  S_j^T of b0 and b1                               (MFMA)
//      phase 2:  O_b1 += V_{j-1}^T P_{j-1,b1}^T  beside  softmax of S_{j,b0}
//      phase 3:  O_b0 += V_j^T P_{j,b0}^T        beside  softmax of S_{j,b1}
//    so the vector work of one block is issued between the matrix
//    instructions of the other (P V of block b1 trails by one tile).  V tiles
//    are read one tile longer than K tiles; both use four LDS buffers and are
//    fetched two tiles ahead with direct loads.
//  * softmax fast path: a row's reference max m is only raised when needed.
//    P~ = exp2(c S - m) is formed with the current m; if every lane's partial
//    row sum stays at or below 2^16 (so no P~ exceeds it) the tile is
//    accepted as is.  Otherwise, or while some row has seen no visible key
//    yet, the block takes the full path (row max, new reference, rescale of
//    O~ and l).  Any reference gives the same O = O~ / l and LSE = m + log2 l,
//    so this changes rounding only.  The row sum is taken in fp32 over the
//    unrounded P~ (a sum of the bf16 values would move the LSE by up to
//    about 1e-3).
//
// Hazards of the inline MFMAs (the compiler does not see them as MFMAs):
//  * the P operand is written by vector instructions just before: two wait
//    states (s_nop 1) precede every inline MFMA;
//  * vector access to the accumulators (rare rescale, epilogue) first waits
//    for all MFMAs in flight (agpr_settle, 24 wait states), and MFMAs after a
//    vector write to them wait 5 wait states (agpr_publish);
//  * all of these are volatile asm statements, which the compiler keeps in
//    program order.
//  * back-to-back accumulation into the same AGPRs needs no wait on gfx950.
#include "miattn_device.h"
#include "miattn_launch.h"

#include <type_traits>

namespace miattn {

namespace {

constexpr float kFastBound = 65536.0f;  // 2^16: largest accepted per-lane partial row sum

// Every statement that touches the accumulator AGPRs names all 128 of them
// as clobbered, so the compiler keeps none of its own values there and
// counts them in the kernel's register allocation.
#define MIATTN_ACC_CLOBBERS \
  "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", \
  "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", \
  "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", \
  "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", \
  "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", \
  "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", \
  "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", \
  "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127"

// acc[IDX] += a * b, accumulator block IDX in AGPRs 16*IDX .. 16*IDX+15.
#define MIATTN_MFMA_AT(LO, HI) \
  __asm__ volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[" #LO ":" #HI "], %0, %1, a[" #LO ":" #HI "]" \
                   :: "v"(a), "v"(b) : MIATTN_ACC_CLOBBERS)
__device__ __forceinline__ void mfma_acc(int idx, bf16x8 a, bf16x8 b) {
  switch (idx) {
    case 0: MIATTN_MFMA_AT(0, 15); break;
    case 1: MIATTN_MFMA_AT(16, 31); break;
    case 2: MIATTN_MFMA_AT(32, 47); break;
    case 3: MIATTN_MFMA_AT(48, 63); break;
    case 4: MIATTN_MFMA_AT(64, 79); break;
    case 5: MIATTN_MFMA_AT(80, 95); break;
    case 6: MIATTN_MFMA_AT(96, 111); break;
    case 7: MIATTN_MFMA_AT(112, 127); break;
    default: break;
  }
}

// x[0..15] = accumulator block IDX (after agpr_settle).
__device__ __forceinline__ void acc_read16(int idx, float (&x)[16]) {
  switch (idx) {
    case 0:
      __asm__ volatile("v_accvgpr_read_b32 %0, a0\n\tv_accvgpr_read_b32 %1, a1\n\tv_accvgpr_read_b32 %2, a2\n\tv_accvgpr_read_b32 %3, a3\n\tv_accvgpr_read_b32 %4, a4\n\tv_accvgpr_read_b32 %5, a5\n\tv_accvgpr_read_b32 %6, a6\n\tv_accvgpr_read_b32 %7, a7\n\tv_accvgpr_read_b32 %8, a8\n\tv_accvgpr_read_b32 %9, a9\n\tv_accvgpr_read_b32 %10, a10\n\tv_accvgpr_read_b32 %11, a11\n\tv_accvgpr_read_b32 %12, a12\n\tv_accvgpr_read_b32 %13, a13\n\tv_accvgpr_read_b32 %14, a14\n\tv_accvgpr_read_b32 %15, a15"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 1:
      __asm__ volatile("v_accvgpr_read_b32 %0, a16\n\tv_accvgpr_read_b32 %1, a17\n\tv_accvgpr_read_b32 %2, a18\n\tv_accvgpr_read_b32 %3, a19\n\tv_accvgpr_read_b32 %4, a20\n\tv_accvgpr_read_b32 %5, a21\n\tv_accvgpr_read_b32 %6, a22\n\tv_accvgpr_read_b32 %7, a23\n\tv_accvgpr_read_b32 %8, a24\n\tv_accvgpr_read_b32 %9, a25\n\tv_accvgpr_read_b32 %10, a26\n\tv_accvgpr_read_b32 %11, a27\n\tv_accvgpr_read_b32 %12, a28\n\tv_accvgpr_read_b32 %13, a29\n\tv_accvgpr_read_b32 %14, a30\n\tv_accvgpr_read_b32 %15, a31"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 2:
      __asm__ volatile("v_accvgpr_read_b32 %0, a32\n\tv_accvgpr_read_b32 %1, a33\n\tv_accvgpr_read_b32 %2, a34\n\tv_accvgpr_read_b32 %3, a35\n\tv_accvgpr_read_b32 %4, a36\n\tv_accvgpr_read_b32 %5, a37\n\tv_accvgpr_read_b32 %6, a38\n\tv_accvgpr_read_b32 %7, a39\n\tv_accvgpr_read_b32 %8, a40\n\tv_accvgpr_read_b32 %9, a41\n\tv_accvgpr_read_b32 %10, a42\n\tv_accvgpr_read_b32 %11, a43\n\tv_accvgpr_read_b32 %12, a44\n\tv_accvgpr_read_b32 %13, a45\n\tv_accvgpr_read_b32 %14, a46\n\tv_accvgpr_read_b32 %15, a47"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 3:
      __asm__ volatile("v_accvgpr_read_b32 %0, a48\n\tv_accvgpr_read_b32 %1, a49\n\tv_accvgpr_read_b32 %2, a50\n\tv_accvgpr_read_b32 %3, a51\n\tv_accvgpr_read_b32 %4, a52\n\tv_accvgpr_read_b32 %5, a53\n\tv_accvgpr_read_b32 %6, a54\n\tv_accvgpr_read_b32 %7, a55\n\tv_accvgpr_read_b32 %8, a56\n\tv_accvgpr_read_b32 %9, a57\n\tv_accvgpr_read_b32 %10, a58\n\tv_accvgpr_read_b32 %11, a59\n\tv_accvgpr_read_b32 %12, a60\n\tv_accvgpr_read_b32 %13, a61\n\tv_accvgpr_read_b32 %14, a62\n\tv_accvgpr_read_b32 %15, a63"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 4:
      __asm__ volatile("v_accvgpr_read_b32 %0, a64\n\tv_accvgpr_read_b32 %1, a65\n\tv_accvgpr_read_b32 %2, a66\n\tv_accvgpr_read_b32 %3, a67\n\tv_accvgpr_read_b32 %4, a68\n\tv_accvgpr_read_b32 %5, a69\n\tv_accvgpr_read_b32 %6, a70\n\tv_accvgpr_read_b32 %7, a71\n\tv_accvgpr_read_b32 %8, a72\n\tv_accvgpr_read_b32 %9, a73\n\tv_accvgpr_read_b32 %10, a74\n\tv_accvgpr_read_b32 %11, a75\n\tv_accvgpr_read_b32 %12, a76\n\tv_accvgpr_read_b32 %13, a77\n\tv_accvgpr_read_b32 %14, a78\n\tv_accvgpr_read_b32 %15, a79"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 5:
      __asm__ volatile("v_accvgpr_read_b32 %0, a80\n\tv_accvgpr_read_b32 %1, a81\n\tv_accvgpr_read_b32 %2, a82\n\tv_accvgpr_read_b32 %3, a83\n\tv_accvgpr_read_b32 %4, a84\n\tv_accvgpr_read_b32 %5, a85\n\tv_accvgpr_read_b32 %6, a86\n\tv_accvgpr_read_b32 %7, a87\n\tv_accvgpr_read_b32 %8, a88\n\tv_accvgpr_read_b32 %9, a89\n\tv_accvgpr_read_b32 %10, a90\n\tv_accvgpr_read_b32 %11, a91\n\tv_accvgpr_read_b32 %12, a92\n\tv_accvgpr_read_b32 %13, a93\n\tv_accvgpr_read_b32 %14, a94\n\tv_accvgpr_read_b32 %15, a95"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 6:
      __asm__ volatile("v_accvgpr_read_b32 %0, a96\n\tv_accvgpr_read_b32 %1, a97\n\tv_accvgpr_read_b32 %2, a98\n\tv_accvgpr_read_b32 %3, a99\n\tv_accvgpr_read_b32 %4, a100\n\tv_accvgpr_read_b32 %5, a101\n\tv_accvgpr_read_b32 %6, a102\n\tv_accvgpr_read_b32 %7, a103\n\tv_accvgpr_read_b32 %8, a104\n\tv_accvgpr_read_b32 %9, a105\n\tv_accvgpr_read_b32 %10, a106\n\tv_accvgpr_read_b32 %11, a107\n\tv_accvgpr_read_b32 %12, a108\n\tv_accvgpr_read_b32 %13, a109\n\tv_accvgpr_read_b32 %14, a110\n\tv_accvgpr_read_b32 %15, a111"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    case 7:
      __asm__ volatile("v_accvgpr_read_b32 %0, a112\n\tv_accvgpr_read_b32 %1, a113\n\tv_accvgpr_read_b32 %2, a114\n\tv_accvgpr_read_b32 %3, a115\n\tv_accvgpr_read_b32 %4, a116\n\tv_accvgpr_read_b32 %5, a117\n\tv_accvgpr_read_b32 %6, a118\n\tv_accvgpr_read_b32 %7, a119\n\tv_accvgpr_read_b32 %8, a120\n\tv_accvgpr_read_b32 %9, a121\n\tv_accvgpr_read_b32 %10, a122\n\tv_accvgpr_read_b32 %11, a123\n\tv_accvgpr_read_b32 %12, a124\n\tv_accvgpr_read_b32 %13, a125\n\tv_accvgpr_read_b32 %14, a126\n\tv_accvgpr_read_b32 %15, a127"
                       : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15]));
      break;
    default: break;
  }
}

// accumulator block IDX = x[0..15]; followed by agpr_publish before any MFMA.
__device__ __forceinline__ void acc_write16(int idx, const float (&x)[16]) {
  switch (idx) {
    case 0:
      __asm__ volatile("v_accvgpr_write_b32 a0, %0\n\tv_accvgpr_write_b32 a1, %1\n\tv_accvgpr_write_b32 a2, %2\n\tv_accvgpr_write_b32 a3, %3\n\tv_accvgpr_write_b32 a4, %4\n\tv_accvgpr_write_b32 a5, %5\n\tv_accvgpr_write_b32 a6, %6\n\tv_accvgpr_write_b32 a7, %7\n\tv_accvgpr_write_b32 a8, %8\n\tv_accvgpr_write_b32 a9, %9\n\tv_accvgpr_write_b32 a10, %10\n\tv_accvgpr_write_b32 a11, %11\n\tv_accvgpr_write_b32 a12, %12\n\tv_accvgpr_write_b32 a13, %13\n\tv_accvgpr_write_b32 a14, %14\n\tv_accvgpr_write_b32 a15, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 1:
      __asm__ volatile("v_accvgpr_write_b32 a16, %0\n\tv_accvgpr_write_b32 a17, %1\n\tv_accvgpr_write_b32 a18, %2\n\tv_accvgpr_write_b32 a19, %3\n\tv_accvgpr_write_b32 a20, %4\n\tv_accvgpr_write_b32 a21, %5\n\tv_accvgpr_write_b32 a22, %6\n\tv_accvgpr_write_b32 a23, %7\n\tv_accvgpr_write_b32 a24, %8\n\tv_accvgpr_write_b32 a25, %9\n\tv_accvgpr_write_b32 a26, %10\n\tv_accvgpr_write_b32 a27, %11\n\tv_accvgpr_write_b32 a28, %12\n\tv_accvgpr_write_b32 a29, %13\n\tv_accvgpr_write_b32 a30, %14\n\tv_accvgpr_write_b32 a31, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 2:
      __asm__ volatile("v_accvgpr_write_b32 a32, %0\n\tv_accvgpr_write_b32 a33, %1\n\tv_accvgpr_write_b32 a34, %2\n\tv_accvgpr_write_b32 a35, %3\n\tv_accvgpr_write_b32 a36, %4\n\tv_accvgpr_write_b32 a37, %5\n\tv_accvgpr_write_b32 a38, %6\n\tv_accvgpr_write_b32 a39, %7\n\tv_accvgpr_write_b32 a40, %8\n\tv_accvgpr_write_b32 a41, %9\n\tv_accvgpr_write_b32 a42, %10\n\tv_accvgpr_write_b32 a43, %11\n\tv_accvgpr_write_b32 a44, %12\n\tv_accvgpr_write_b32 a45, %13\n\tv_accvgpr_write_b32 a46, %14\n\tv_accvgpr_write_b32 a47, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 3:
      __asm__ volatile("v_accvgpr_write_b32 a48, %0\n\tv_accvgpr_write_b32 a49, %1\n\tv_accvgpr_write_b32 a50, %2\n\tv_accvgpr_write_b32 a51, %3\n\tv_accvgpr_write_b32 a52, %4\n\tv_accvgpr_write_b32 a53, %5\n\tv_accvgpr_write_b32 a54, %6\n\tv_accvgpr_write_b32 a55, %7\n\tv_accvgpr_write_b32 a56, %8\n\tv_accvgpr_write_b32 a57, %9\n\tv_accvgpr_write_b32 a58, %10\n\tv_accvgpr_write_b32 a59, %11\n\tv_accvgpr_write_b32 a60, %12\n\tv_accvgpr_write_b32 a61, %13\n\tv_accvgpr_write_b32 a62, %14\n\tv_accvgpr_write_b32 a63, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 4:
      __asm__ volatile("v_accvgpr_write_b32 a64, %0\n\tv_accvgpr_write_b32 a65, %1\n\tv_accvgpr_write_b32 a66, %2\n\tv_accvgpr_write_b32 a67, %3\n\tv_accvgpr_write_b32 a68, %4\n\tv_accvgpr_write_b32 a69, %5\n\tv_accvgpr_write_b32 a70, %6\n\tv_accvgpr_write_b32 a71, %7\n\tv_accvgpr_write_b32 a72, %8\n\tv_accvgpr_write_b32 a73, %9\n\tv_accvgpr_write_b32 a74, %10\n\tv_accvgpr_write_b32 a75, %11\n\tv_accvgpr_write_b32 a76, %12\n\tv_accvgpr_write_b32 a77, %13\n\tv_accvgpr_write_b32 a78, %14\n\tv_accvgpr_write_b32 a79, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 5:
      __asm__ volatile("v_accvgpr_write_b32 a80, %0\n\tv_accvgpr_write_b32 a81, %1\n\tv_accvgpr_write_b32 a82, %2\n\tv_accvgpr_write_b32 a83, %3\n\tv_accvgpr_write_b32 a84, %4\n\tv_accvgpr_write_b32 a85, %5\n\tv_accvgpr_write_b32 a86, %6\n\tv_accvgpr_write_b32 a87, %7\n\tv_accvgpr_write_b32 a88, %8\n\tv_accvgpr_write_b32 a89, %9\n\tv_accvgpr_write_b32 a90, %10\n\tv_accvgpr_write_b32 a91, %11\n\tv_accvgpr_write_b32 a92, %12\n\tv_accvgpr_write_b32 a93, %13\n\tv_accvgpr_write_b32 a94, %14\n\tv_accvgpr_write_b32 a95, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 6:
      __asm__ volatile("v_accvgpr_write_b32 a96, %0\n\tv_accvgpr_write_b32 a97, %1\n\tv_accvgpr_write_b32 a98, %2\n\tv_accvgpr_write_b32 a99, %3\n\tv_accvgpr_write_b32 a100, %4\n\tv_accvgpr_write_b32 a101, %5\n\tv_accvgpr_write_b32 a102, %6\n\tv_accvgpr_write_b32 a103, %7\n\tv_accvgpr_write_b32 a104, %8\n\tv_accvgpr_write_b32 a105, %9\n\tv_accvgpr_write_b32 a106, %10\n\tv_accvgpr_write_b32 a107, %11\n\tv_accvgpr_write_b32 a108, %12\n\tv_accvgpr_write_b32 a109, %13\n\tv_accvgpr_write_b32 a110, %14\n\tv_accvgpr_write_b32 a111, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    case 7:
      __asm__ volatile("v_accvgpr_write_b32 a112, %0\n\tv_accvgpr_write_b32 a113, %1\n\tv_accvgpr_write_b32 a114, %2\n\tv_accvgpr_write_b32 a115, %3\n\tv_accvgpr_write_b32 a116, %4\n\tv_accvgpr_write_b32 a117, %5\n\tv_accvgpr_write_b32 a118, %6\n\tv_accvgpr_write_b32 a119, %7\n\tv_accvgpr_write_b32 a120, %8\n\tv_accvgpr_write_b32 a121, %9\n\tv_accvgpr_write_b32 a122, %10\n\tv_accvgpr_write_b32 a123, %11\n\tv_accvgpr_write_b32 a124, %12\n\tv_accvgpr_write_b32 a125, %13\n\tv_accvgpr_write_b32 a126, %14\n\tv_accvgpr_write_b32 a127, %15"
                       :: "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]) : MIATTN_ACC_CLOBBERS);
      break;
    default: break;
  }
}

// Wait until every MFMA into the accumulators has completed (before vector
// reads of them), and until vector writes to them are visible (before MFMAs).
__device__ __forceinline__ void agpr_settle() { __asm__ volatile("s_nop 15\n\ts_nop 7"); }
__device__ __forceinline__ void agpr_publish() { __asm__ volatile("s_nop 4"); }


}  // namespace

template <int D, bool CAUSAL, bool VARLEN, bool KPAD>
__global__ void __launch_bounds__(256, 1) fwd_w4_kernel(AttnArgs a, int n_qtiles) {
  constexpr int NW = 4;
  constexpr int BC = 64;
  constexpr int BR = NW * 64;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  constexpr int LPT = BC * CPR / NT;  // direct loads per thread per tensor and tile
  constexpr int NLD = 2 * LPT;        // per tile, K and V
  constexpr int NBUF = 4;
  constexpr int NPV = 4 * DB;         // P V MFMAs per block and tile
  constexpr int EPC = 32 / NPV;       // softmax elements per lane handled beside one of them
  static_assert(LPT * NT == BC * CPR, "tile chunks must divide evenly");
  static_assert(NLD < 16, "vmcnt field of 4 bits");

  __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NBUF][TILE];
  __shared__ uint8_t s_valid[NBUF][BC];
  __shared__ uint32_t s_anypad[NBUF];

  int bh, tile;
  wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, CAUSAL, bh, tile);  // causal: heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<VARLEN>(a, b, h, D);
  const int q_tile0 = tile * BR;
  if (q_tile0 >= sv.len) return;  // uniform across the workgroup, before any barrier

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int q_wave0 = q_tile0 + wave * 64;  // block qb covers rows q_wave0 + 32 qb .. + 31
  const int kv_len = sv.len;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.kv_base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.kv_base;

  // A negative scale is handled by flipping the sign of Q once.
  float c = a.scale_log2;
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  c = fabsf(c);

  bf16x8 qf[2][KS];  // loaded in the prologue
  float m[2], l[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m[qb] = kNegInf;
    l[qb] = 0.f;
  }
  {
    const float zero[16] = {};
#pragma unroll
    for (int idx = 0; idx < 2 * DB; ++idx) acc_write16(idx, zero);
    agpr_publish();
  }

  const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
  const int ntiles = (kv_end + BC - 1) / BC;
  // both blocks of a wave end on the same key tile (BC divides 64)
  const int jw_last = CAUSAL ? min(ntiles - 1, (q_wave0 + 63) / BC) : ntiles - 1;

  // Direct-load sources: LDS chunk p = i*NT + tid of a tile holds row p / CPR,
  // logical chunk (p % CPR) ^ swz(row).  Rows past the sequence repeat its
  // last row (finite values, masked).
  int src_row[LPT], src_col[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int pch = i * NT + tid;
    const int row = pch / CPR;
    src_row[i] = row;
    src_col[i] = ((pch % CPR) ^ swz<D>(row)) << 3;
  }
  // Load number n (0 .. NLD-1) of this thread for tile j: K for even n, V for
  // odd n, chunk n / 2.
  auto issue_part = [&](int j, int n) {
    const int i = n >> 1;
    const int key = min(j * BC + src_row[i], kv_len - 1);
    const int64_t off = (int64_t)key * sv.kv_stride + src_col[i];
    if (n & 1) lds_dma16(vp + off, sV[j % NBUF] + (i * NT + wave * 64) * 8);
    else lds_dma16(kp + off, sK[j % NBUF] + (i * NT + wave * 64) * 8);
  };
  auto issue = [&](int j) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) issue_part(j, n);
  };
  // Key-validity flags of a tile, by wave 0: loaded raw before the tile's
  // direct loads are issued, converted and stored at the end of the step.
  uint32_t rvalid = 1u;
  int rkey = 0;
  auto load_flags = [&](int j) {
    if constexpr (KPAD) {
      if (wave == 0) {
        rkey = j * BC + lane;
        rvalid = a.key_valid[sv.tok0 + min(rkey, kv_len - 1)];
      }
    }
  };
  auto store_flags = [&](int j) {
    if constexpr (KPAD) {
      if (wave == 0) {
        const uint32_t ok = (rkey >= kv_len || rvalid != 0u) ? 1u : 0u;  // keys past the end are masked anyway
        s_valid[j % NBUF][lane] = (uint8_t)ok;
        const bool any = wave_any(ok == 0u);
        if (lane == 0) s_anypad[j % NBUF] = any ? 1u : 0u;
      }
    }
  };

  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = swz_off<D>(l32, ks * 16 + hi * 8);
  const int tr_r = hi * 4 + ((lane >> 2) & 3);
  const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int voff[2][DB];
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);

  f32x16 s[2][2];  // [block][32-key half] scores of the current tile
  u32x4 p0[4];     // packed P of block 0, current tile
  u32x4 p1[4];     // packed P of block 1, previous tile (its P V trails)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p0[i] = u32x4{0u, 0u, 0u, 0u};
    p1[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // Phase 1: S^T of both blocks.  K operands are read two k-steps ahead of
  // their MFMAs (one wave per SIMD: nothing else hides the LDS latency); the
  // loads of tile j+2 go between the MFMAs.
  auto mma_s = [&](int j, bool fetch) {
    const uint16_t* kt = sK[j % NBUF];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[qb][kb] = f32x16{};
    bf16x8 ka[3][2];
    auto kread = [&](int ks, bf16x8 (&dst)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dst[kb] = as_bf16x8(*(const u32x4*)(kt + kb * 32 * D + koff[ks]));
    };
    kread(0, ka[0]);
    kread(1, ka[1]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 2 < KS) kread(ks + 2, ka[(ks + 2) % 3]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[0][kb] = mfma_bf16(ka[ks % 3][kb], qf[0][ks], s[0][kb]);
        s[1][kb] = mfma_bf16(ka[ks % 3][kb], qf[1][ks], s[1][kb]);
      }
      if (fetch) {
#pragma unroll
        for (int n = ks * NLD / KS; n < (ks + 1) * NLD / KS; ++n) issue_part(j + 2, n);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Masking of a tile's scores for both blocks (diagonal, end, padded keys);
  // returns the exponent multiplier (1 once the scores carry the scale).
  auto mask = [&](int j) -> float {
    const int kt0 = j * BC;
    bool need_mask = kt0 + BC > kv_len;
    if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > q_wave0);
    if (KPAD) need_mask = need_mask || (s_anypad[j % NBUF] != 0u);
    if (!need_mask) return c;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = pin_in_branch(q_wave0 + qb * 32 + l32);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const int key = kt0 + kl;
          bool vis = key < kv_len;
          if (CAUSAL) vis = vis && key <= qi;
          if (KPAD) vis = vis && s_valid[j % NBUF][kl] != 0;
          s[qb][kb][r] = vis ? s[qb][kb][r] * c : kNegInf;
        }
    }
    return 1.f;
  };
  // Softmax elements [i*EPC, (i+1)*EPC) of block qb with reference mu:
  // exp2, bf16 packing into pw and the row-sum update.
  auto sm_part = [&](int qb, int i, float cc, float mu, u32x4 (&pw)[4], float& rs) {
#pragma unroll
    for (int e = 0; e < EPC; e += 2) {
      const int idx = i * EPC + e;
      const int kb = idx >> 4;
      const int r = idx & 15;
      const float e0 = fast_exp2(__builtin_fmaf(s[qb][kb][r], cc, -mu));
      const float e1 = fast_exp2(__builtin_fmaf(s[qb][kb][r + 1], cc, -mu));
      pw[kb * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(e0, e1);
      rs += e0;
      rs += e1;
    }
  };
  // Full path for block qb: row max, new reference, exp2 and sums; returns
  // the rescale factor of its O~ (1 when nothing changes).
  auto softmax_full = [&](int qb, float cc, u32x4 (&pw)[4]) -> float {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
    mx = wave_max_halves(mx) * cc;
    const float m_new = mx > m[qb] ? mx : m[qb];
    const bool dead = m_new == kNegInf;  // no visible key yet for this row
    const float alpha = dead ? 1.f : fast_exp2(m[qb] - m_new);
    const float mu = dead ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < NPV; ++i) sm_part(qb, i, cc, mu, pw, rs);
    l[qb] = alpha * l[qb] + rs;
    m[qb] = m_new;
    return alpha;
  };
  // O~ of block qb times alpha (the rare full-path case).
  auto rescale = [&](int qb, float alpha) {
    if (wave_any(alpha != 1.f)) {
      const float a_ = pin_in_branch(alpha);
      agpr_settle();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float x[16];
        acc_read16(qb * DB + db, x);
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] *= a_;
        acc_write16(qb * DB + db, x);
      }
      agpr_publish();
    }
  };
  // After the fast path of block qb (partial sums rs): accept it, or redo
  // the block on the full path.
  auto finish = [&](int qb, float cc, float rs, u32x4 (&pw)[4]) {
    if (wave_any(!(rs <= kFastBound))) {
      const float alpha = softmax_full(qb, cc, pw);
      rescale(qb, alpha);
    } else {
      l[qb] += rs;
    }
  };
  // V^T operand of P V MFMA number i (key step kb*2+t, column block db).
  auto v_operand = [&](const uint16_t* vt, int i) -> bf16x8 {
    const int db = i % DB;
    const int kt = i / DB;  // = kb * 2 + t
    const uint16_t* v0 = vt + kt * 16 * D;
    return join_u32x2(lds_read_tr16(v0 + voff[0][db]), lds_read_tr16(v0 + voff[1][db]));
  };
  // P V of one block (tile jv, packed P pp, accumulators of block acc_blk).
  // With SM, the fast-path softmax of block qb is issued between its MFMAs
  // as a three-stage pipeline over chunks of EPC elements (exponent argument
  // two MFMAs ahead, exp2 one ahead, packing and sums), so that no vector
  // instruction waits on the one before it; returns the partial row sum.
  // V operands are read three MFMAs ahead.
  auto pv_mma = [&](auto sm_c, int jv, int acc_blk, const u32x4 (&pp)[4], int qb, float cc,
                    u32x4 (&pw)[4]) -> float {
    constexpr bool SM = decltype(sm_c)::value;
    constexpr int PF = 3;
    const uint16_t* vt = sV[jv % NBUF];
    const float mu = m[qb];
    float rsa = 0.f, rsb = 0.f;
    bf16x8 va[NPV];
    float t[NPV][EPC];
    auto stage_arg = [&](int c) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int idx = c * EPC + e;
        t[c][e] = __builtin_fmaf(s[qb][idx >> 4][idx & 15], cc, -mu);
      }
    };
    auto stage_exp = [&](int c) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) t[c][e] = fast_exp2(t[c][e]);
    };
    auto stage_pack = [&](int c) {
#pragma unroll
      for (int e = 0; e < EPC; e += 2) {
        const int idx = c * EPC + e;
        const int kb = idx >> 4;
        const int r = idx & 15;
        uint32_t w = pack_bf16x2(t[c][e], t[c][e + 1]);
        rsa += t[c][e];
        rsb += t[c][e + 1];
        // keep this stage between the MFMAs it was written beside (the
        // compiler would otherwise sink it towards the first use)
        __asm__ volatile("" : "+v"(w), "+v"(rsa), "+v"(rsb));
        pw[kb * 2 + (r >> 3)][(r & 7) >> 1] = w;
      }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) va[i] = v_operand(vt, i);
    if constexpr (SM) {
      stage_arg(0);
      stage_arg(1);
      stage_exp(0);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + PF < NPV) va[i + PF] = v_operand(vt, i + PF);
      mfma_acc(acc_blk * DB + i % DB, va[i], as_bf16x8(pp[i / DB]));
      if constexpr (SM) {
        if (i + 2 < NPV) stage_arg(i + 2);
        if (i + 1 < NPV) stage_exp(i + 1);
        stage_pack(i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return rsa + rsb;
  };

  // Tile j: phases 1-3.  Block 1's P V trails by one tile; at j = 0 its
  // packed P is still zero, so that product (on tile 0's V) adds nothing.
  // The fast path runs unconditionally: while a row has no finite reference
  // it yields an infinite or NaN sum, which sends the block to the full path.
  auto work = [&](int j, bool fetch) {
    mma_s(j, fetch);
    __builtin_amdgcn_sched_barrier(0);
    const float cc = mask(j);
    __builtin_amdgcn_sched_barrier(0);
    const float rs0 = pv_mma(std::true_type{}, j > 0 ? j - 1 : 0, 1, p1, 0, cc, p0);
    finish(0, cc, rs0, p0);
    __builtin_amdgcn_sched_barrier(0);
    const float rs1 = pv_mma(std::true_type{}, j, 0, p0, 1, cc, p1);
    finish(1, cc, rs1, p1);
    __builtin_amdgcn_sched_barrier(0);
  };
  // P V of block 1 for its last tile (nothing beside it).
  auto trailing_pv1 = [&](int jv) {
    u32x4 unused[4];
    pv_mma(std::false_type{}, jv, 1, p1, 1, 1.f, unused);
  };
  // End of tile j: this wave's loads of tile j+1 have landed (those of j+2
  // may still be in flight), then the barrier.
  auto end_tile = [&](int j) {
    if (j + 2 < ntiles) store_flags(j + 2);
    if (j + 2 < ntiles) barrier_vmem_n<NLD>();
    else barrier_vmem_n<0>();
  };

  // Prologue: tiles 0 and 1 in flight, then this wave's Q rows; one wait.
  load_flags(0);
  store_flags(0);
  if (ntiles > 1) {
    load_flags(1);
    store_flags(1);
  }
  issue(0);
  if (ntiles > 1) issue(1);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = q_wave0 + qb * 32 + l32;
    const uint32_t keep = qi < kv_len ? 0xffffffffu : 0u;
    const uint16_t* qrow = qp + (int64_t)min(qi, kv_len - 1) * sv.tok_stride + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = as_bf16x8((*(const u32x4*)(qrow + ks * 16) & keep) ^ qsign);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  barrier_vmem_n<0>();

  // Every wave passes ntiles barriers: tiles 0..jw_last with work, then
  // tiles in which it only fetches for the others (the first of them also
  // finishes block 1's trailing P V).
  for (int j = 0; j <= jw_last; ++j) {
    const bool fetch = j + 2 < ntiles;
    if (fetch) load_flags(j + 2);
    work(j, fetch);
    end_tile(j);
  }
  for (int j = jw_last + 1; j < ntiles; ++j) {
    const bool fetch = j + 2 < ntiles;
    if (fetch) {
      load_flags(j + 2);
      issue(j + 2);
    }
    if (j == jw_last + 1) trailing_pv1(jw_last);
    end_tile(j);
  }
  if (jw_last == ntiles - 1) trailing_pv1(jw_last);

  // Epilogue: O = O~ / l, LSE = ln 2 * (m + log2 l); a row that saw no
  // visible key gets O = 0 and LSE = -inf.
  agpr_settle();
  uint16_t* __restrict__ op = (uint16_t*)a.o + sv.base;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = wave_sum_halves(l[qb]);
    const int qi = q_wave0 + qb * 32 + l32;
    if (qi < sv.len) {
      const bool dead = (m[qb] == kNegInf) || !(lt > 0.f);
      const float inv = dead ? 0.f : 1.f / lt;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float x[16];
        acc_read16(qb * DB + db, x);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                     pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
          *(u32x2*)(op + (int64_t)qi * sv.tok_stride + db * 32 + g * 8 + hi * 4) = w;
        }
      }
      if (hi == 0) a.lse[sv.row_base + qi] = dead ? kNegInf : (m[qb] + fast_log2(lt)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool KPAD>
static hipError_t launch_fwd_w4_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BR = 4 * 64;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_w4_kernel<D, CAUSAL, VARLEN, KPAD>), dim3((unsigned)blocks), dim3(256), 0, stream, a,
                     n_qtiles);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_fwd_w4(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
  if (varlen) {
    if (causal) return kpad ? launch_fwd_w4_t<D, true, true, true>(a, s) : launch_fwd_w4_t<D, true, true, false>(a, s);
    return kpad ? launch_fwd_w4_t<D, false, true, true>(a, s) : launch_fwd_w4_t<D, false, true, false>(a, s);
  }
  return causal ? launch_fwd_w4_t<D, true, false, false>(a, s) : launch_fwd_w4_t<D, false, false, false>(a, s);
}

hipError_t launch_fwd_w4_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream) {
  const bool kpad = varlen && a.key_valid != nullptr;
  if (d == 128) return dispatch_fwd_w4<128>(a, causal, varlen, kpad, stream);
  if (d == 64) return dispatch_fwd_w4<64>(a, causal, varlen, kpad, stream);
  return hipErrorInvalidValue;
}

}  // namespace miattn
