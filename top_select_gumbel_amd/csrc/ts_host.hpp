// ts_host.hpp -- host helpers shared by the sources of libtopselect.so.
#pragma once

namespace tsh {

// Records a thread-local message (printf-style) for ts_last_error() and returns `code`.
int fail(int code, const char* fmt, ...);
// TS_OK with the current device in *dev_out if it is a gfx950, else TS_ERR_UNSUPPORTED.
int check_device(int* dev_out);
const char* last_error();

}  // namespace tsh
