// Host build of the library's quantiser helpers (w8a8_int8_post_amd/csrc/
// sq_device.h), for a CPU test that replays the arithmetic the kernels run
// -- the row-step Markstein quotient, the saturating form for a step fixed in
// advance, and the plain IEEE division for steps outside [2^-96, 2^96] --
// and compares the codes with the oracle's IEEE quotient.  Test
// infrastructure: nothing in the library includes or links this file.
#include "sq_device.h"

extern "C" {

// codes[i] for (v[i], step[i]) as a kernel takes them: the fast quotient
// where the step allows it, else the division; sat != 0 selects the
// saturating form used with a static (given) step.
void hq_codes(const float* v, const float* step, long n, int sat, signed char* codes) {
    for (long i = 0; i < n; ++i) {
        const sq::RowStep q = sq::given_step(step[i]);
        int c;
        if (q.fast)
            c = sat ? sq::quant_code<true, true>(v[i], q) : sq::quant_code<true, false>(v[i], q);
        else
            c = sq::quant_code<false>(v[i], q);
        codes[i] = (signed char)c;
    }
}

// Number of fp32 bit patterns u in [lo, hi) whose code differs from the
// definition (roundf, halves away from zero, clamped to +-127).
long hq_rounding_mismatches(unsigned lo, unsigned long hi) {
    long bad = 0;
    for (unsigned long u = lo; u < hi; ++u) {
        float t;
        const unsigned b = (unsigned)u;
        __builtin_memcpy(&t, &b, 4);
        float r = __builtin_roundf(t);
        r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
        bad += sq::code_from_quotient(t) != (int)r;
    }
    return bad;
}

// The row step absmax / 127 as the kernels compute it.
float hq_row_step(float absmax) { return sq::quant_step(absmax); }

}
