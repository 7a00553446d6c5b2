// Internal to libw4a16: the current HIP device's properties the entry points check and use,
// queried once per device.
#ifndef W4A16_DEVICE_H
#define W4A16_DEVICE_H

namespace w4a16_detail {

struct DeviceInfo {
    bool queried = false;
    bool gfx950 = false;
    int cus = 0;      // compute units
};

// Fills *out for the current device.  W4A16_OK, W4A16_EUNSUPPORTED (not gfx950) or
// W4A16_EHIP (no current device, or its properties could not be read).
__attribute__((visibility("hidden"))) int current_device(DeviceInfo *out);

}  // namespace w4a16_detail

#endif  // W4A16_DEVICE_H
