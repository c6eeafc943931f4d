// Status strings and version of libdflash2 (the C ABI declared in dflash2.h).
#include "common.hpp"

extern "C" const char* dflash2_status_string(int code) {
  switch (code) {
    case DFLASH2_OK: return "ok";
    case DFLASH2_EINVAL: return "invalid argument (null pointer, bad size or inconsistent shape)";
    case DFLASH2_EUNSUPPORTED: return "unsupported shape, type or alignment";
    case DFLASH2_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case DFLASH2_EHIP: return "kernel launch failed";
    case DFLASH2_ST_NONFINITE: return "status: nonfinite selector score or NaN chosen by the greedy chain";
    case DFLASH2_ST_BADTOKEN: return "status: index out of range or proposal/slot mismatch";
    case DFLASH2_ST_ZEROMASS: return "status: sampling row without mass";
    case DFLASH2_ST_BADPROB: return "status: probability outside [0, 1], or sampling on a bf16 target";
    case DFLASH2_ST_BADTEMP: return "status: invalid temperature (treated as greedy)";
    case DFLASH2_ST_RINGLOST: return "status: rewind past the positions the ring holds";
    case DFLASH2_ST_BADCOUNT: return "status: ring update count out of range (clamped)";
    default: return "unknown code";
  }
}

extern "C" int dflash2_version(void) { return 100; }
