// Host build of the grouped GEMM epilogue's MXFP4 / MXFP8 block encoder
// (mx_scale_byte and mx_encode from the library's common.hpp), so a CPU test
// can compare it with the oracle over every bf16 pattern and every scale
// byte a block can reach.  Compiled by tests/test_encoder_host.py with
// `hipcc -x hip --offload-host-only`; nothing here runs on a GPU.
#include <stdint.h>

#include "../../moe_expert_grouped_gemm_amd/csrc/common.hpp"

using namespace ptgg;

// Blocks of 32 consecutive bf16 values (x holds nblocks * 32), encoded the
// way the SwiGLU -> MXFP4 epilogue does: amax over the magnitudes' bits,
// E = mx_scale_byte(amax), every code by mx_encode(value, E).
//   fmt 0 (E4M3): q [nblocks * 32] bytes;  fmt 1 (E2M1): q [nblocks * 16],
//   element 2i in the low nibble of byte i.  s [nblocks] scale bytes.
extern "C" int ptgg_host_mx_encode_blocks(const uint16_t *x, int64_t nblocks, int fmt, uint8_t *q, uint8_t *s)
{
    if (fmt != 0 && fmt != 1) return -1;
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint16_t *v = x + b * 32;
        uint32_t amax = 0;
        for (int i = 0; i < 32; ++i) amax = amax > (v[i] & 0x7FFFu) ? amax : (v[i] & 0x7FFFu);
        if (fmt == 0) {
            const uint32_t E = mx_scale_byte<8>(amax);
            s[b] = (uint8_t)E;
            for (int i = 0; i < 32; ++i) q[b * 32 + i] = (uint8_t)mx_encode<0>(v[i], E);
        } else {
            const uint32_t E = mx_scale_byte<2>(amax);
            s[b] = (uint8_t)E;
            for (int i = 0; i < 16; ++i)
                q[b * 16 + i] = (uint8_t)(mx_encode<1>(v[2 * i], E) | (mx_encode<1>(v[2 * i + 1], E) << 4));
        }
    }
    return 0;
}
